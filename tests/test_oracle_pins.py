"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: each compares it with a closed
form, a textbook or library routine (torch SDPA on the CPU), a hand-worked
example, an invariant, or a constructed case whose outcome is predicted by
hand.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle.compare import check_list, replay_walk
from synth import config, make, shrink, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _shape(**kw):
    base = dict(batch=1, q_heads=1, kv_heads=1, seq_len=512, head_dim=32, block=64,
                causal=True, scale=0.0, dtype="f32")
    base.update(kw)
    return O.Shape(**base)


def _rand(n, d, seed, dtype="f32"):
    x = np.random.default_rng(seed).standard_normal((n, d), dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


# ------------------------------------------------------------------ rounding / pooling

def test_bf16_round_ties_to_even():
    # IEEE 754 round-to-nearest-even at 8 significand bits (bfloat16).
    one = 1.0
    cases = {
        one: one,
        one + 2.0 ** -8: one,                              # halfway, even below
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,              # halfway, even above
        one + 2.0 ** -8 + 2.0 ** -20: one + 2.0 ** -7,     # above halfway
        one + 2.0 ** -9: one,                              # below halfway
        -(one + 2.0 ** -8): -one,
        3.0 + 2.0 ** -7: 3.0,                             # halfway at exponent 1, even below
    }
    x = np.array(list(cases.keys()), dtype=np.float32)
    got = O.round_to_dtype(x, "bf16")
    want = np.array(list(cases.values()), dtype=np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g", [1, 2, 4, 16, 32])
def test_pool_mean_exact_on_integer_rows(dtype, g):
    # Integer rows whose group sums are multiples of g: every partial sum is exact in
    # fp32 and the mean is a small integer, exact in bf16.  The pooled row must be it.
    rng = np.random.default_rng(g)
    n, d = 8 * g, 16
    x = rng.integers(-20, 21, size=(n, d)).astype(np.float32)
    x3 = x.reshape(n // g, g, d)
    x3[:, -1, :] -= (x3.sum(axis=1) % g)                   # make group sums divisible by g
    want = x3.astype(np.float64).mean(axis=1)
    got = O.pool_rows(x, g, O.POOL_MEAN, dtype)
    assert np.array_equal(got.astype(np.float64), want)


def test_pool_mean_close_to_true_mean():
    x = _rand(1024, 64, 3)
    for g in (4, 32):
        got = O.pool_rows(x, g, O.POOL_MEAN, "bf16").astype(np.float64)
        mean = x.astype(np.float64).reshape(-1, g, 64).mean(axis=1)
        # fp32 summation error plus half a bf16 ulp
        bound = g * 2.0 ** -24 * np.abs(x).reshape(-1, g, 64).sum(axis=1) / g + np.abs(mean) * 2.0 ** -8 + 1e-30
        assert np.all(np.abs(got - mean) <= bound * 1.01)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_mean_sums_rows_in_ascending_order(dtype):
    # The pooled row is the fp32 sum of the g rows taken in ascending order.  Column 0 holds
    # 2^24, 1, 1, -2^24: in fp32, 2^24 + 1 rounds back to 2^24 (ties to even), so the
    # ascending sum is 2^24, 2^24, 0 -> mean 0.  Summed in descending order it would be
    # -2^24 + 1 + 1 + 2^24 = 2 (all partial sums exact) -> 0.5, and pairwise
    # (2^24 + 1) + (1 - 2^24) = 2^24 - (2^24 - 1) = 1 -> 0.25.  Column 1 is the same rows
    # reversed: ascending gives 2 -> 0.5.  All three values are exact in bf16.
    x = np.array([[2.0 ** 24, -(2.0 ** 24)], [1.0, 1.0], [1.0, 1.0], [-(2.0 ** 24), 2.0 ** 24]],
                 dtype=np.float32)
    got = O.pool_rows(x, 4, O.POOL_MEAN, dtype)
    assert got.tolist() == [[0.0, 0.5]]


def test_pool_stride_and_identity():
    x = _rand(256, 8, 4)
    assert np.array_equal(O.pool_rows(x, 8, O.POOL_STRIDE, "f32"), x[::8])
    assert np.array_equal(O.pool_rows(x, 1, O.POOL_MEAN, "f32"), x)


# ------------------------------------------------------------------ proxy

def test_proxy_g1_is_blockmax_of_true_scores():
    # With g = 1 the proxy sees the real queries and keys: P[r, j] is the max of the
    # true attention logits of row r over the visible keys of block j, and the HRM
    # block of row r is the block holding its exact argmax.
    sh = _shape(seq_len=256, block=32, head_dim=16)
    q = _rand(256, 16, 5)
    k = _rand(256, 16, 6)
    logits = (torch.from_numpy(q).double() @ torch.from_numpy(k).double().T) / 4.0
    logits = logits.masked_fill(torch.ones(256, 256, dtype=torch.bool).triu(1), float("-inf")).numpy()
    kp = O.KapParams(budget=1.0, pool=1)
    for i in (0, 3, 7):
        P = O.proxy_block_scores(q, k, i, sh, 1)
        for rr in range(32):
            r = i * 32 + rr
            for j in range(8):
                want = logits[r, j * 32:(j + 1) * 32].max()
                assert P[rr, j] == pytest.approx(want, rel=1e-12, abs=1e-12) or (np.isinf(want) and np.isinf(P[rr, j]))
        u = O.kap_unit(P, i, sh, kp)
        arg_blocks = {int(np.argmax(logits[i * 32 + rr])) // 32 for rr in range(32)}
        assert set(np.nonzero(u["hrm"])[0].tolist()) == arg_blocks


def test_proxy_maxnorm_invariants():
    sh = _shape(seq_len=2048, block=64, head_dim=32, dtype="bf16")
    q = _rand(2048, 32, 7, "bf16")
    k = _rand(2048, 32, 8, "bf16")
    kp = O.KapParams(budget=0.3)
    rb = 64 // kp.g(sh)
    for u in O.kap_head(q, k, sh, kp, blocks=[0, 5, 31]):
        c = np.exp(u["P"] - u["rowmax"][:, None])
        assert np.all(c > 0) and np.all(c <= 1)
        assert np.all((c == 1).sum(axis=1) == 1)         # one maximum per pooled row
        assert np.all(u["S"] <= rb + 1e-12)
        assert 1 <= u["hrm_cnt"] <= rb
        assert np.all(u["S"][u["hrm"]] >= 1.0)            # an HRM block holds some row's 1


def test_kap_worked_example():
    """Hand-worked example (tests/golden/kap_worked_example.json).

    B = 2, g = 1, D = 2, scale 1.  Query block 3 holds rows 6 = (1,0) and 7 = (0,1),
    so row 6 scores key c by k_c[0] and row 7 by k_c[1]; key 7 is hidden from row 6.
    Block maxima: row 6 -> [1, 3, 1, 2], row 7 -> [0, 1, 2, 5].  Row maxima sit in
    blocks 1 and 3 (HRM).  MaxNorm: row 6 -> e^[-2, 0, -2, -1], row 7 -> e^[-5, -4, -3, 0].
    Sum: [e^-2+e^-5, 1+e^-4, e^-2+e^-3, e^-1+1]; HRM first by score: 3, 1; then 2, 0.
    Zero query rows tie every score, so the lowest block wins the HRM flag and ties
    keep ascending block order.
    """
    ex = json.load(open(os.path.join(GOLDEN, "kap_worked_example.json")))
    s = ex["shape"]
    sh = _shape(seq_len=s["seq_len"], block=s["block"], head_dim=s["head_dim"], scale=s["scale"])
    q = np.array(ex["q"], dtype=np.float32)
    k = np.array(ex["k"], dtype=np.float32)
    e = ex["expected"]
    full = O.kap_head(q, k, sh, O.KapParams(budget=1.0, pool=1))
    assert np.array_equal(full[3]["P"], np.array(e["block3"]["P"], dtype=np.float64))
    assert np.allclose(full[3]["S"], e["block3"]["S_sum"], rtol=1e-15)
    assert sorted(np.nonzero(full[3]["hrm"])[0].tolist()) == sorted(e["block3"]["hrm"])
    assert full[3]["list"].tolist() == e["block3"]["order_sum"]
    assert full[2]["list"].tolist() == e["block2"]["order_sum"]
    assert full[1]["list"].tolist() == e["block1"]["order_sum"]
    assert full[0]["list"].tolist() == e["block0"]["order_sum"]
    mx = O.kap_head(q, k, sh, O.KapParams(budget=1.0, pool=1, agg_mode=O.AGG_MAX))
    assert mx[3]["list"].tolist() == e["block3"]["order_max"]
    half = O.kap_head(q, k, sh, O.KapParams(budget=0.5, pool=1))
    assert half[3]["list"].tolist() == e["block3"]["list_rho_0.5"]
    assert half[2]["list"].tolist() == e["block2"]["list_rho_0.5"]
    tq = O.kap_head(q, k, sh, O.KapParams(budget=0.75, pool=1))
    assert tq[3]["list"].tolist() == e["block3"]["list_rho_0.75"]
    # cumulative mass on block 3: order 3, 1, 2, 0 with S = 1.368, 1.018, 0.185, 0.142 (total
    # 2.713); prefix sums 1.368, 2.386, 2.571, 2.713.  mass 0.5 needs 1.357 -> 1 block;
    # mass 0.8 needs 2.171 -> 2 blocks; mass 0.93 needs 2.523 -> 3 blocks, unless the budget
    # (k = 2 at rho 0.5) caps it first.
    cm = lambda mass, rho=1.0: O.kap_head(q, k, sh, O.KapParams(budget=rho, pool=1, sel_mode=O.SEL_CUMMASS,
                                                                mass=mass))[3]["list"].tolist()
    assert cm(0.5) == [3]
    assert cm(0.8) == [3, 1]
    assert cm(0.93) == [3, 1, 2]
    assert cm(0.93, rho=0.5) == [3, 1]
    assert cm(1.0) == [3, 1, 2, 0]


@pytest.mark.parametrize("mass,want", [(0.5, [0]), (0.75, [0, 1]), (0.74, [0, 1]), (0.76, [0, 1, 2])])
def test_cummass_stops_where_the_prefix_reaches_the_goal(mass, want):
    # Block scores built to be exact: four pooled rows whose logits are 0 in one block and
    # -1000 elsewhere (exp(-1000) is 0 in double), maxima in blocks 0, 0, 1, 2.  MaxNorm then
    # gives S = [2, 1, 1, 0] and HRM = {0, 1, 2}; the order is 0, 1, 2, 3 (HRM first, S
    # descending, ties by ascending block).  Total 4.  The list is the shortest prefix whose
    # score sum reaches mass * 4: a prefix that meets the goal exactly (2 at mass 0.5, 3 at
    # mass 0.75) ends the list there.
    sh = _shape(seq_len=256, block=64, head_dim=8)
    P = np.full((4, 4), -1000.0)
    for r, j in enumerate([0, 0, 1, 2]):
        P[r, j] = 0.0
    u = O.kap_unit(P, 3, sh, O.KapParams(budget=1.0, pool=16, sel_mode=O.SEL_CUMMASS, mass=mass))
    assert u["S"].tolist() == [2.0, 1.0, 1.0, 0.0]
    assert u["list"].tolist() == want
    assert u["k"] == len(want)


def test_forced_sink_and_diag_flags():
    """Forced HRM flags on the worked example, by hand.

    Block 3 (HRM {1, 3}; S = 1.368, 1.018, 0.185, 0.142 for blocks 3, 1, 2, 0): a forced
    sink adds block 0 to the HRM group, which goes first by S, so the order becomes
    3, 1, 0, 2; the diagonal (block 3) is HRM already, so forcing it changes nothing.
    Block 2 (zero query rows: every visible block scores S = 2, the lowest, block 0, holds
    both row maxima): a forced diagonal adds block 2, which ties block 0 on S and follows
    it in block order, then block 1.
    """
    ex = json.load(open(os.path.join(GOLDEN, "kap_worked_example.json")))
    s = ex["shape"]
    sh = _shape(seq_len=s["seq_len"], block=s["block"], head_dim=s["head_dim"], scale=s["scale"])
    q = np.array(ex["q"], dtype=np.float32)
    k = np.array(ex["k"], dtype=np.float32)
    run = lambda **kw: O.kap_head(q, k, sh, O.KapParams(budget=1.0, pool=1, **kw))
    sink = run(force_sink=True)
    assert sink[3]["list"].tolist() == [3, 1, 0, 2]
    assert sorted(np.nonzero(sink[3]["hrm"])[0].tolist()) == [0, 1, 3]
    diag = run(force_diag=True)
    assert diag[3]["list"].tolist() == [3, 1, 2, 0]
    assert diag[2]["list"].tolist() == [0, 2, 1]
    assert sorted(np.nonzero(diag[2]["hrm"])[0].tolist()) == [0, 2]
    both = run(force_sink=True, force_diag=True)
    assert both[3]["list"].tolist() == [3, 1, 0, 2]
    assert both[0]["list"].tolist() == [0]


@pytest.mark.parametrize("causal", [True, False])
def test_select_invariants(causal):
    sh = _shape(seq_len=4096, block=128, head_dim=32, dtype="bf16", causal=causal)
    q = _rand(4096, 32, 9, "bf16")
    k = _rand(4096, 32, 10, "bf16")
    for rho in (0.1, 0.37, 1.0):
        for u in O.kap_head(q, k, sh, O.KapParams(budget=rho), blocks=[0, 1, 17, 31]):
            n = u["n"]
            assert n == (u["P"].shape[1])
            assert u["k"] == min(n, max(1, math.ceil(rho * n)))
            lst = u["list"]
            assert len(set(lst.tolist())) == len(lst) == u["k"]
            assert lst.min() >= 0 and lst.max() < n
            if rho == 1.0:
                assert sorted(lst.tolist()) == list(range(n))
            h = u["hrm"][lst]
            nh = min(u["hrm_cnt"], u["k"])
            assert h[:nh].all() and not h[nh:].any()      # HRM prefix
            key = [(int(u["hrm"][j]), u["S"][j], -int(j)) for j in lst]
            assert key == sorted(key, reverse=True)


def test_budget_count():
    assert O.budget_count(0.1, 1024) == 103
    assert O.budget_count(0.05, 1024) == 52
    assert O.budget_count(0.1, 1000) == 100
    assert O.budget_count(0.05, 20) == 1
    assert O.budget_count(0.01, 5) == 1
    assert O.budget_count(1.0, 7) == 7


def test_planted_blocks_rank_first():
    # Config 1's structure (salient key blocks along each KV head's query direction
    # plus a sink block 0): the planted blocks visible to a query block outrank all
    # background blocks, and the first list entry is a planted one.
    cfg = shrink(config(1), 4096, q_heads=4, kv_heads=1, n_salient=4)
    x = make(cfg)
    sh = O.Shape(1, 4, 1, 4096, 128, 128, True, 0.0, "bf16")
    kp = O.KapParams(budget=1.0)
    kk = x["k"][0, 0]
    # recover the planted blocks: their keys are nearly parallel within the block
    norms = np.linalg.norm(kk.reshape(32, 128, 128).mean(axis=1), axis=1)
    planted = set(np.nonzero(norms > 10)[0].tolist())
    assert 0 in planted and len(planted) == 5
    for h in range(4):
        for u, i in zip(O.kap_head(x["q"][0, h], kk, sh, kp, blocks=[3, 20, 31]), [3, 20, 31]):
            vis = [j for j in planted if j <= i]
            assert int(u["list"][0]) in planted
            assert set(u["list"][:len(vis)].tolist()) == set(vis)


# ------------------------------------------------------------------ OSK

def _sdpa(q, k, v, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).double()[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)[0, 0].numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("perm", [False, True])
def test_full_budget_no_skip_is_dense_attention(causal, perm):
    # rho = rho' = 1, skip off: the sparse method is dense softmax attention.
    sh = _shape(seq_len=512, block=64, head_dim=32, causal=causal)
    q, k, v = (_rand(512, 32, s) for s in (11, 12, 13))
    ref = _sdpa(q, k, v, causal)
    # LSE: the library's logsumexp of the scaled, masked logits (natural log)
    logits = torch.from_numpy(q).double() @ torch.from_numpy(k).double().T / math.sqrt(32)
    if causal:
        logits = logits.masked_fill(torch.ones(512, 512, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(logits, dim=1).numpy()
    kp = O.KapParams(budget=1.0)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF)
    rng = np.random.default_rng(0)
    for u, i in zip(O.kap_head(q, k, sh, kp), range(sh.nb)):
        lst = rng.permutation(u["list"]) if perm else u["list"]
        w = O.osk_unit(q, k, v, i, lst, u["k"], sh, op)
        assert (w["status"][: u["k"]] == 1).all()
        assert np.allclose(w["out"], ref[i * 64:(i + 1) * 64], atol=1e-12, rtol=0)
        assert np.allclose(w["out_walk"], ref[i * 64:(i + 1) * 64], atol=1e-12, rtol=0)
        assert np.allclose(w["lse"], ref_lse[i * 64:(i + 1) * 64], atol=1e-12, rtol=0)
        assert np.allclose(w["lse_walk"], ref_lse[i * 64:(i + 1) * 64], atol=1e-12, rtol=0)
    o_dense, lse_dense = O.dense_attention(q, k, v, sh)
    assert np.allclose(o_dense, ref, atol=1e-12, rtol=0)
    assert np.allclose(lse_dense, ref_lse, atol=1e-12, rtol=0)


def test_gqa_head_mapping_matches_sdpa():
    # Query head h reads KV head h // G (consecutive grouping).
    G, n, d = 4, 256, 16
    rng = np.random.default_rng(14)
    q = rng.standard_normal((G * 2, n, d)).astype(np.float32)
    k = rng.standard_normal((2, n, d)).astype(np.float32)
    v = rng.standard_normal((2, n, d)).astype(np.float32)
    tq = torch.from_numpy(q).double()[None]
    tk = torch.from_numpy(k).double()[None].repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).double()[None].repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy()
    sh = _shape(seq_len=n, block=64, head_dim=d, q_heads=8, kv_heads=2)
    for h in range(8):
        res = O.run_head(q[h], k[h // G], v[h // G], sh, O.KapParams(budget=1.0),
                         O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF))
        out = np.concatenate([r["osk"]["out"] for r in res])
        assert np.allclose(out, ref[h], atol=1e-12)


def test_order_invariance_of_walk():
    # Without skipping, the walk's online-softmax result does not depend on the
    # visiting order (technical summary, section 2.1).
    sh = _shape(seq_len=1024, block=64, head_dim=32)
    q, k, v = (_rand(1024, 32, s) for s in (15, 16, 17))
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF)
    i = 12
    lst = np.array([12, 0, 5, 7, 11, 3])
    rng = np.random.default_rng(1)
    q_blk = q[i * 64:(i + 1) * 64]
    base = O.osk_walk(q_blk, k, v, i, lst, len(lst), sh, op)
    for _ in range(5):
        w = O.osk_walk(q_blk, k, v, i, rng.permutation(lst), len(lst), sh, op)
        assert np.allclose(w["out_walk"], base["out_walk"], atol=1e-12, rtol=0)
        assert np.allclose(w["lse_walk"], base["lse_walk"], atol=1e-12, rtol=0)


def _concentrated(n=4096):
    cfg = shrink(config(1), n, q_heads=4, kv_heads=1, n_salient=6)
    cfg.update(salient_gain=12.0, q_noise=0.2)
    return cfg


def test_walk_equals_closed_form_with_skipping():
    x = make(_concentrated())
    sh = O.Shape(1, 4, 1, 4096, 128, 128, True, 0.0, "bf16")
    res = O.run_head(x["q"][0, 1], x["k"][0, 0], x["v"][0, 0], sh, O.KapParams(budget=0.5),
                     O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_MASS, skip_param=1e-3))
    n_skip = 0
    for r in res:
        w = r["osk"]
        assert np.allclose(w["out_walk"], w["out"], atol=1e-12, rtol=0)
        assert np.allclose(w["lse_walk"], w["lse"], atol=1e-12, rtol=0)
        n_skip += int((w["status"] == 2).sum())
    assert n_skip > 0                                     # the structured input does skip


def test_constant_v_gives_constant_output():
    sh = _shape(seq_len=1024, block=64, head_dim=32)
    q, k = _rand(1024, 32, 18), _rand(1024, 32, 19)
    vrow = np.linspace(-1, 1, 32).astype(np.float32)
    v = np.tile(vrow, (1024, 1))
    for r in O.run_head(q, k, v, sh, O.KapParams(budget=0.3), O.OskParams(tight_budget=0.15)):
        assert np.allclose(r["osk"]["out"], vrow[None, :], atol=1e-12)


def test_one_hot_block_v_reads_off_computed_set():
    # V[c, block(c)] = 1: output column j is the attention mass on block j, so the
    # computed blocks are exactly the non-zero columns and the columns sum to 1.
    sh = _shape(seq_len=1024, block=64, head_dim=64)
    q, k = _rand(1024, 64, 20), _rand(1024, 64, 21)
    v = np.zeros((1024, 64), np.float32)
    v[np.arange(1024), np.arange(1024) // 64] = 1.0
    for r in O.run_head(q, k, v, sh, O.KapParams(budget=0.5), O.OskParams(tight_budget=0.25)):
        out = r["osk"]["out"]
        comp = set(r["osk"]["computed"].tolist())
        nz = set(np.nonzero(np.abs(out).max(axis=0) > 0)[0].tolist())
        assert nz == comp
        assert np.allclose(out.sum(axis=1), 1.0, atol=1e-12)


def _dominance_case(first: bool):
    # Every query row is 8 e_0, scale 1/8, so row r scores key c by k_c[0].
    # Block 2's keys score 40; all other keys score N(0,1): a >= 30 gap.
    sh = _shape(seq_len=1024, block=64, head_dim=64, scale=1.0 / 8)
    q = np.zeros((1024, 64), np.float32)
    q[:, 0] = 8.0
    k = _rand(1024, 64, 22)
    k[128:192, 0] = 40.0
    v = _rand(1024, 64, 23)
    i = 15
    others = [0, 1, 3, 4, 5, 6, 7, 15]
    lst = np.array(([2] + others) if first else (others + [2]))
    return sh, q, k, v, i, lst


def test_dominant_block_first_skips_everything_after():
    sh, q, k, v, i, lst = _dominance_case(first=True)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=1e-3)
    w = O.osk_unit(q, k, v, i, lst, len(lst), sh, op)
    assert w["status"].tolist() == [1] + [2] * (len(lst) - 1)
    opm = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MAXDIFF, skip_param=-20.0)
    w = O.osk_unit(q, k, v, i, lst, len(lst), sh, opm)
    assert w["status"].tolist() == [1] + [2] * (len(lst) - 1)


@pytest.mark.parametrize("second,want", [(-1.0, [1, 1]), (-3.0, [1, 2])])
def test_maxdiff_compares_the_local_max_with_the_running_max_only(second, want):
    # MAXDIFF skips a block iff every row's local max is at most tau above the running max,
    # whatever the running denominator.  Query rows e_0, scale 1: row r scores key c by
    # k_c[0].  Block 0: every key scores 0, so after it m = 0 and l = 64 (ln l = 4.16).
    # Block 1: every key scores `second`.  With tau = -2, a local max of -1 (-1 > -2) is
    # computed and one of -3 is skipped; a statistic that also subtracted ln l would skip both.
    sh = _shape(seq_len=256, block=64, head_dim=8, scale=1.0)
    q = np.zeros((256, 8), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((256, 8), np.float32)
    k[64:128, 0] = second
    v = _rand(256, 8, 31)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MAXDIFF, skip_param=-2.0)
    w = O.osk_unit(q, k, v, 2, np.array([0, 1]), 2, sh, op)
    assert w["status"].tolist() == want


def test_dominant_block_last_skips_nothing():
    sh, q, k, v, i, lst = _dominance_case(first=False)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=1e-3)
    w = O.osk_unit(q, k, v, i, lst, len(lst), sh, op)
    assert w["status"].tolist() == [1] * len(lst)


# ------------------------------------------------------------------ visible keys nv in the MASS test

EPS = 1e-3


def _nv_diag_case():
    """Causal, two blocks of 64 (head dim 64, scale 1); query block 1 walks [0, 1].

    Block 0's keys are zero: every row of block 1 scores 0 on all 64 of them, so after
    the first (computed) block m = 0 and l = 64 on every row.  On the diagonal block row
    r sees keys 0..r (nv = r + 1).  Query row 0 of block 1 is x e_0 and key 0 of block 1
    is e_0 - 30 e_1; rows r >= 1 are e_1 and keys 1..63 are -30 e_1.  So row 0's local
    maximum is x (key 0 is all it sees) and every other row's is -30.  The MASS statistic
    of row r is m_loc - m + ln nv - ln l:
        row 0:        x + ln 1 - ln 64
        rows r >= 1:  -30 + ln(r + 1) - ln 64   (at most -30)
    With x = ln eps + ln(64)/2, row 0 sits ln(64)/2 below the threshold ln eps and every
    other row more than 23 below: the block is skipped.  Counting all 64 keys of the
    block on row 0 would put it ln(64)/2 above the threshold instead.
    """
    B, D = 64, 64
    sh = _shape(seq_len=2 * B, block=B, head_dim=D, scale=1.0)
    q = np.zeros((2 * B, D), np.float32)
    k = np.zeros((2 * B, D), np.float32)
    v = _rand(2 * B, D, 31)
    x = math.log(EPS) + math.log(B) / 2
    q[B, 0] = x
    q[B + 1:, 1] = 1.0
    k[B, 0], k[B, 1] = 1.0, -30.0
    k[B + 1:, 1] = -30.0
    return sh, q, k, v


def test_mass_counts_visible_keys_on_the_diagonal_block():
    sh, q, k, v = _nv_diag_case()
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=EPS)
    w = O.osk_unit(q, k, v, 1, np.array([0, 1]), 2, sh, op)
    assert w["status"].tolist() == [1, 2]
    # the deciding row is row 0, at ln(64)/2 below the threshold
    d, _ = w["margins"][1]
    x = float(q[64, 0])                                   # ln eps + ln(64)/2 as stored (fp32)
    assert abs(d - (x - math.log(64) - math.log(EPS))) < 1e-12, d
    assert abs(d + math.log(64) / 2) < 1e-6
    # only block 0 computed, all its logits 0: every row's output is the mean of its V rows
    assert np.allclose(w["out"], v[:64].astype(np.float64).mean(axis=0)[None, :], atol=1e-12)
    assert np.allclose(w["lse"], math.log(64), atol=1e-12)


def test_mass_counts_the_keys_of_a_ragged_last_block():
    """Non-causal, 80 tokens at block 64: block 1 holds 16 keys.  Query block 0 walks [0, 1].
    Block 0's keys are zero (m = 0, l = 64 on every row); every query row is e_0 and every
    key of block 1 is y e_0, so each row scores y on the 16 keys that exist.  MASS statistic:
    y + ln 16 - ln 64.  With y = ln eps + ln(4)/2 every row sits ln(4)/2 below the threshold
    and the block is skipped; counting 64 keys would put every row ln(4)/2 above it."""
    B, D, n = 64, 32, 80
    sh = _shape(seq_len=n, block=B, head_dim=D, scale=1.0, causal=False)
    q = np.zeros((n, D), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((n, D), np.float32)
    k[B:, 0] = math.log(EPS) + math.log(4) / 2
    v = _rand(n, D, 32)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=EPS)
    w = O.osk_unit(q, k, v, 0, np.array([0, 1]), 2, sh, op)
    assert w["status"].tolist() == [1, 2]
    d, _ = w["margins"][1]
    y = float(k[B, 0])                                    # ln eps + ln(4)/2 as stored (fp32)
    assert abs(d - (y + math.log(16) - math.log(64) - math.log(EPS))) < 1e-12, d
    assert abs(d + math.log(4) / 2) < 1e-6
    assert np.allclose(w["out"], v[:64].astype(np.float64).mean(axis=0)[None, :], atol=1e-12)


# ------------------------------------------------------------------ KV page remap

@pytest.mark.parametrize("skip", [O.SKIP_OFF, O.SKIP_MASS])
def test_page_table_walk_equals_walk_in_logical_order(skip):
    """[Summary] §2.3: blocks are reached by remapping KV pages.  K and V stored with their
    pages in a permuted order, walked with the table that maps each logical block to its
    page, must give the walk over K and V in logical order with no table: the same
    statuses, decision margins, output and LSE (bitwise: the same numbers in the same
    order).  Query rows are 8 e_0 at scale 1/8 and block 2's keys score 40, so with block
    2 listed first the skip test fires on the blocks after it."""
    B, nb, D = 64, 8, 32
    sh = _shape(seq_len=nb * B, block=B, head_dim=D, scale=1.0 / 8)
    rng = np.random.default_rng(41)
    q = _rand(nb * B, D, 42)
    q[:, 0] = 8.0
    k = _rand(nb * B, D, 43)
    k[2 * B:3 * B, 0] = 40.0
    v = _rand(nb * B, D, 44)
    page = np.roll(np.arange(nb), 3)[rng.permutation(nb)]   # logical block j lives in page[j]
    assert (page != np.arange(nb)).any()
    kp, vp = np.empty_like(k), np.empty_like(v)
    for j in range(nb):
        kp[page[j] * B:(page[j] + 1) * B] = k[j * B:(j + 1) * B]
        vp[page[j] * B:(page[j] + 1) * B] = v[j * B:(j + 1) * B]
    op = O.OskParams(tight_budget=1.0, skip_mode=skip, skip_param=EPS)
    differs = skipped = 0
    for i in range(nb):
        lst = rng.permutation(i + 1)
        if i >= 2:
            lst = np.concatenate([[2], lst[lst != 2]])
        ref = O.osk_unit(q, k, v, i, lst, len(lst), sh, op)
        got = O.osk_unit(q, kp, vp, i, lst, len(lst), sh, op, page_table=page)
        assert np.array_equal(got["status"], ref["status"])
        assert got["margins"] == ref["margins"]
        assert np.array_equal(got["out"], ref["out"]) and np.array_equal(got["lse"], ref["lse"])
        skipped += int((ref["status"] == 2).sum())
        # the table matters: the permuted storage read in logical order gives another result
        bad = O.osk_unit(q, kp, vp, i, lst, len(lst), sh, op)
        differs += int(not np.allclose(bad["out"], ref["out"]))
    assert differs >= nb - 1
    assert (skipped > 0) == (skip == O.SKIP_MASS)


def test_eps_to_zero_is_skip_off():
    cfg = shrink(config(2), 4096, q_heads=4, kv_heads=1)
    x = make(cfg)
    sh = O.Shape(1, 4, 1, 4096, 128, 128, True, 0.0, "bf16")
    kp = O.KapParams(budget=0.5)
    a = O.run_head(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], sh, kp,
                   O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_MASS, skip_param=1e-300))
    b = O.run_head(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], sh, kp,
                   O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_OFF))
    for ra, rb_ in zip(a, b):
        assert np.array_equal(ra["osk"]["status"], rb_["osk"]["status"])
        assert np.array_equal(ra["osk"]["out"], rb_["osk"]["out"])


@pytest.mark.parametrize("cap_mode", [O.COMPUTED, O.VISITED])
def test_cap_counts(cap_mode):
    cfg = shrink(config(2), 4096, q_heads=4, kv_heads=1)
    x = make(cfg)
    sh = O.Shape(1, 4, 1, 4096, 128, 128, True, 0.0, "bf16")
    kp = O.KapParams(budget=0.6)
    for skip in (O.SKIP_OFF, O.SKIP_MASS):
        op = O.OskParams(tight_budget=0.3, cap_mode=cap_mode, skip_mode=skip)
        for r in O.run_head(x["q"][0, 2], x["k"][0, 0], x["v"][0, 0], sh, kp, op):
            w, u = r["osk"], r["kap"]
            kpr = min(u["k"], O.budget_count(0.3, u["n"]))
            st = w["status"]
            if cap_mode == O.COMPUTED:
                assert w["n_comp"] == min(kpr, int((st[:u["k"]] != 2).sum()) if skip else u["k"])
                assert w["n_comp"] == kpr or w["visited"] == u["k"]
            else:
                assert w["visited"] == kpr
            if skip == O.SKIP_OFF:
                assert w["n_comp"] == kpr
            assert (st[w["visited"]:] == 0).all()


# ------------------------------------------------------------------ brute force

def _brute_kap(q, k, B, g, rho, scale):
    """Element-by-element re-derivation on a tiny input (loops, no numpy vector ops).
    n need not be a multiple of B or g: the last pooled row averages what exists
    (times 1/g), the last block has fewer rows and keys."""
    n, d = len(q), len(q[0])
    def pooled(x, r):
        acc = [np.float32(0.0)] * d
        for t in range(g):
            if r * g + t >= n:
                break
            for e in range(d):
                acc[e] = np.float32(acc[e] + np.float32(x[r * g + t][e]))
        return [float(np.float32(a / np.float32(g))) for a in acc]
    npool = -(-n // g)
    qp = [pooled(q, r) for r in range(npool)]
    kp = [pooled(k, r) for r in range(npool)]
    rb = B // g
    nb = -(-n // B)
    lists = []
    for i in range(nb):
        cand = list(range(i + 1))
        P = []
        for rr in range(rb):
            r = i * rb + rr
            if r >= npool:
                break
            row = []
            for j in cand:
                best = -math.inf
                for tt in range(rb):
                    t = j * rb + tt
                    if t <= r and t < npool:
                        best = max(best, scale * sum(qp[r][e] * kp[t][e] for e in range(d)))
                row.append(best)
            P.append(row)
        S = [0.0] * len(cand)
        hrm = [False] * len(cand)
        for row in P:
            mx = max(row)
            hrm[row.index(mx)] = True
            for j in cand:
                S[j] += math.exp(row[j] - mx)
        order = sorted(cand, key=lambda j: (not hrm[j], -S[j], j))
        kk = min(len(cand), max(1, math.ceil(rho * len(cand))))
        lists.append(order[:kk])
    return lists


@pytest.mark.parametrize("n", [64, 58, 49])
def test_brute_force_tiny_kap(n):
    d, B, g = 4, 16, 4
    q = _rand(n, d, 24)
    k = _rand(n, d, 25)
    sh = _shape(seq_len=n, block=B, head_dim=d)
    got = [u["list"].tolist() for u in O.kap_head(q, k, sh, O.KapParams(budget=0.6, pool=g))]
    want = _brute_kap(q.tolist(), k.tolist(), B, g, 0.6, 1.0 / math.sqrt(d))
    assert got == want


# ------------------------------------------------------------------ comparator self-tests

def _unit_for_compare():
    sh = _shape(seq_len=4096, block=128, head_dim=32, dtype="bf16")
    q = _rand(4096, 32, 26, "bf16")
    k = _rand(4096, 32, 27, "bf16")
    return O.kap_head(q, k, sh, O.KapParams(budget=0.5), blocks=[31])[0]


def test_comparator_accepts_oracle_and_rejects_planted_mistakes():
    u = _unit_for_compare()
    k = u["k"]
    lst = list(u["list"]) + [-1] * 3
    ok, msg = check_list(u, lst, k, u["hrm_cnt"], u["score"])
    assert ok, msg
    # swap two well-separated entries in the non-HRM part
    h = min(u["hrm_cnt"], k)
    bad = list(lst)
    bad[h], bad[k - 1] = bad[k - 1], bad[h]
    assert not check_list(u, bad, k, u["hrm_cnt"])[0]
    # drop the last entry in favour of the best excluded one... of the worst excluded
    excl = sorted(set(range(u["n"])) - set(u["list"].tolist()), key=lambda j: u["S"][j])
    bad = list(lst)
    bad[k - 1] = excl[0]
    assert not check_list(u, bad, k, u["hrm_cnt"])[0]
    assert not check_list(u, lst, k - 1, u["hrm_cnt"])[0]
    assert not check_list(u, lst, k, u["hrm_cnt"] + 5)[0]
    sc = np.array(u["score"]).copy()
    sc[0] *= 1.001
    assert not check_list(u, lst, k, u["hrm_cnt"], sc)[0]


def _hand_unit(budget):
    # Four pooled rows of query block 5 (six candidate blocks), logits chosen by hand: row maxima in
    # blocks 0, 2, 3 = 4 (an exact tie) and 0.  Definite HRM {0, 2}; possible HRM {0, 2, 3, 4};
    # the oracle flags 3 (lowest index).  S ~ [2.027, 0.046, 1.033, 1.015, 1.013, 0.043], so the
    # full order is 0, 2, 3 (HRM by S), then 4, 1, 5.
    P = np.array([[5.0, 1.0, 0.0, 0.5, 0.2, 0.1],
                  [1.0, 0.5, 6.0, 0.3, 0.2, 0.4],
                  [0.1, 0.2, 0.3, 4.0, 4.0, 0.5],
                  [7.0, 0.3, 0.2, 0.1, 0.4, 0.6]])
    sh = _shape(seq_len=384, block=64, head_dim=8)
    return O.kap_unit(P, 5, sh, O.KapParams(budget=budget, pool=16))


@pytest.mark.parametrize("budget,gpu,cnt,hrm,msg", [
    (1.0, [0, 2, 3, 4, 1, 5], 6, 3, "ok"),                       # the oracle's own list
    (1.0, [0, 2, 4, 3, 1, 5], 6, 3, "ok"),                       # the other side of the row-2 tie
    (0.3, [0, 2], 2, 3, "ok"),
    (0.6, [0, 2, 3, 4, 1], 5, 3, "count"),                       # one entry too many
    (0.6, [0, 2, 3, 4, 1, -1], 4, 3, "padding"),                 # an entry past the count
    (0.6, [0, 2, 3, 6, -1, -1], 4, 3, "index out of candidate"),  # block 6 is no candidate
    (0.6, [0, 2, 3, 3, -1, -1], 4, 3, "duplicate"),
    (0.6, [0, 2, 3, 4, -1, -1], 4, 1, "hrm count"),              # fewer than the definite two
    (0.6, [0, 2, 3, 4, -1, -1], 4, 5, "hrm count"),              # more than the possible four
    (1.0, [0, 2, 1, 3, 4, 5], 6, 3, "position 2 block 1 flagged HRM"),
    (1.0, [0, 3, 4, 2, 1, 5], 6, 3, "position 3 block 2 not flagged HRM"),
    (0.6, [0, 3, 4, 1, -1, -1], 4, 2, "excluded block 2 is HRM"),
    (0.3, [0, 3], 2, 2, "excluded HRM count"),
    (0.3, [0, 3], 2, 3, "excluded HRM block 2 outranks"),
])
def test_comparator_rejects_each_planted_mistake_with_its_own_check(budget, gpu, cnt, hrm, msg):
    u = _hand_unit(budget)
    assert u["list"].tolist() == [0, 2, 3, 4, 1, 5][:u["k"]]
    assert u["hrm"].tolist() == [True, False, True, True, False, False]
    ok, got = check_list(u, gpu, cnt, hrm)
    assert ok == (msg == "ok") and got.startswith(msg), got


def test_comparator_accepts_band_ties():
    u = _unit_for_compare()
    # perturb the oracle's S so two adjacent non-HRM entries tie within the band
    h = min(u["hrm_cnt"], u["k"])
    a, b = u["list"][h], u["list"][h + 1]
    u["S"][b] = u["S"][a] * (1 - 1e-7)
    lst = list(u["list"])
    lst[h], lst[h + 1] = lst[h + 1], lst[h]
    assert check_list(u, lst, u["k"], u["hrm_cnt"])[0]


def test_replay_rejects_statuses_that_are_no_decision():
    sh, q, k, v, i, lst = _dominance_case(first=True)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=1e-3)
    fn = lambda forced: O.osk_unit(q, k, v, i, lst, len(lst), sh, op, forced=forced)
    good = [1] + [2] * (len(lst) - 1)
    assert replay_walk(fn, good)[0]
    # a position the walk reached reported as not reached
    ok, _, msg, _ = replay_walk(fn, good[:-1] + [0])
    assert not ok and msg.startswith("status at position"), msg
    # a status past the end of the list
    ok, _, msg, _ = replay_walk(fn, good + [1])
    assert not ok and msg.startswith("gpu status beyond list"), msg


def test_replay_forces_only_ambiguous_decisions():
    sh, q, k, v, i, lst = _dominance_case(first=True)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MASS, skip_param=1e-3)
    fn = lambda forced: O.osk_unit(q, k, v, i, lst, len(lst), sh, op, forced=forced)
    ok, w, msg, _ = replay_walk(fn, [1] + [2] * (len(lst) - 1))
    assert ok, msg
    # a GPU that computed block 1 instead of skipping it is wrong: the margin is ~30
    ok, w, msg, _ = replay_walk(fn, [1, 1] + [2] * (len(lst) - 2))
    assert not ok
    # a decision right on the threshold may go either way: put MAXDIFF's tau exactly
    # at position 1's statistic, then a GPU that computes there is accepted
    opm = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MAXDIFF, skip_param=-20.0)
    d, _ = O.osk_unit(q, k, v, i, lst, len(lst), sh, opm)["margins"][1]
    on_thr = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_MAXDIFF, skip_param=-20.0 + d)
    fn2 = lambda forced: O.osk_unit(q, k, v, i, lst, len(lst), sh, on_thr, forced=forced)
    assert fn2({})["status"][1] == 2
    flipped = fn2({1: False})["status"]
    assert flipped[1] == 1
    ok, w, msg, forced = replay_walk(fn2, flipped)
    assert ok and forced == {1: False}, msg


def test_score_only_order_differs_from_hrm_first():
    """Hand-worked: two pooled rows with block maxima A = [5, 4.9, 0, 0], B = [0, 4.9, 5, 0].
    HRM blocks are 0 (row A) and 2 (row B), each with S = 1 + e^-5; block 1 is the
    runner-up of both rows, S = 2 e^-0.1 = 1.81, but holds no row maximum; block 3 has
    S = 2 e^-5.  HRM first: 0, 2 (tied S, lower j first), then 1, 3.  By S alone: 1, 0, 2, 3.
    """
    sh = _shape(seq_len=8, block=2, head_dim=2, causal=False)
    P = np.array([[5.0, 4.9, 0.0, 0.0], [0.0, 4.9, 5.0, 0.0]])
    hf = O.kap_unit(P, 3, sh, O.KapParams(budget=1.0, pool=1))
    sc = O.kap_unit(P, 3, sh, O.KapParams(budget=1.0, pool=1, order_mode=O.ORDER_SCORE))
    assert np.allclose(hf["S"], [1 + math.exp(-5), 2 * math.exp(-0.1), 1 + math.exp(-5), 2 * math.exp(-5)])
    assert hf["list"].tolist() == [0, 2, 1, 3]
    assert sc["list"].tolist() == [1, 0, 2, 3]
    assert hf["hrm_cnt"] == sc["hrm_cnt"] == 2
    half = O.kap_unit(P, 3, sh, O.KapParams(budget=0.5, pool=1, order_mode=O.ORDER_SCORE))
    assert half["list"].tolist() == [1, 0]


def test_group_vote_equals_block_vote_without_skipping_and_is_finer_with_it():
    # Skip OFF: the per-group walk computes the same blocks as the block walk.  With the
    # skip test, groups of 32 rows skip blocks that one outlier row of the whole block
    # would have vetoed (the "bucket effect"), so more is skipped on this input.  Each
    # group's output equals the closed form over its own computed set.
    x = make(_concentrated())
    sh = O.Shape(1, 4, 1, 4096, 128, 128, True, 0.0, "bf16")
    kp = O.KapParams(budget=0.5)
    units = O.kap_head(x["q"][0, 0], x["k"][0, 0], sh, kp)
    more = 0
    for i, u in enumerate(units):
        for skip in (O.SKIP_OFF, O.SKIP_MASS):
            opb = O.OskParams(tight_budget=0.5, skip_mode=skip)
            opg = O.OskParams(tight_budget=0.5, skip_mode=skip, vote_rows=32)
            wb = O.osk_unit(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], i, u["list"], u["k"], sh, opb)
            wg = O.osk_unit(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], i, u["list"], u["k"], sh, opg)
            assert wg["status"].shape == (4, len(u["list"]))
            assert np.allclose(wg["out_walk"], wg["out"], atol=1e-12)
            if skip == O.SKIP_OFF:
                for g in range(4):
                    assert np.array_equal(wg["status"][g], wb["status"])
                assert np.allclose(wg["out"], wb["out"], atol=1e-12)
            else:
                more += int((wg["status"] == 2).sum()) - 4 * int((wb["status"] == 2).sum())
    assert more > 0   # finer votes skip more on this input


@pytest.mark.parametrize("n,causal", [(1000, True), (777, True), (1000, False)])
def test_ragged_length_full_budget_is_dense(n, causal):
    # block 64 does not divide n: the last block is partial; at full budget without
    # skipping the method is still dense attention (torch SDPA, fp64).
    sh = _shape(seq_len=n, block=64, head_dim=32, causal=causal)
    q, k, v = (_rand(n, 32, s) for s in (30, 31, 32))
    ref = _sdpa(q, k, v, causal)
    res = O.run_head(q, k, v, sh, O.KapParams(budget=1.0),
                     O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF))
    assert len(res) == -(-n // 64)
    out = np.concatenate([r["osk"]["out"] for r in res])
    assert out.shape == (n, 32)
    assert np.allclose(out, ref, atol=1e-12)
    o_d, _ = O.dense_attention(q, k, v, sh)
    assert np.allclose(o_d, ref, atol=1e-12)


def test_ragged_pool_sums_existing_rows():
    x = np.arange(10 * 4, dtype=np.float32).reshape(10, 4)
    p = O.pool_rows(x, 4, O.POOL_MEAN, "f32")
    assert p.shape == (3, 4)
    assert np.array_equal(p[:2], x[:8].reshape(2, 4, 4).sum(axis=1) / 4)
    assert np.array_equal(p[2], (x[8] + x[9]) / 4)        # partial group: existing rows, same scale
    assert np.array_equal(O.pool_rows(x, 4, O.POOL_STRIDE, "f32"), x[::4])


def test_proxy_g1_ragged_is_blockmax_of_true_scores():
    # g = 1 on a ragged length: the last block has 26 rows and 26 keys; P of its rows
    # is the block max of the true logits over the keys that exist.
    n, B = 250, 32
    sh = _shape(seq_len=n, block=B, head_dim=16)
    q = _rand(n, 16, 7)
    k = _rand(n, 16, 8)
    logits = (torch.from_numpy(q).double() @ torch.from_numpy(k).double().T) / 4.0
    logits = logits.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf")).numpy()
    P = O.proxy_block_scores(q, k, 7, sh, 1)
    assert P.shape == (n - 7 * B, 8)
    for rr in range(n - 7 * B):
        r = 7 * B + rr
        for j in range(8):
            want = logits[r, j * B:min((j + 1) * B, n)].max()
            assert P[rr, j] == pytest.approx(want, rel=1e-12, abs=1e-12) or (np.isinf(want) and np.isinf(P[rr, j]))


@pytest.mark.parametrize("n", [4096 - 88, 4096 - 120])
def test_ragged_group_vote(n):
    # Last block of 40 (or 8) rows: row groups 1.. (or all but the first) hold fewer
    # than 32 rows or none.  Skip OFF: every group that has rows walks like the whole
    # block; an empty group takes no part (all statuses 0, nothing computed).
    x = make(_concentrated())
    q, k, v = (np.ascontiguousarray(x[t][0, 0, :n]) for t in ("q", "k", "v"))
    sh = O.Shape(1, 4, 1, n, 128, 128, True, 0.0, "bf16")
    i = sh.nb - 1
    u = O.kap_head(q, k, sh, O.KapParams(budget=0.5), blocks=[i])[0]
    rows = n - i * 128
    opb = O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_OFF)
    opg = O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_OFF, vote_rows=32)
    wb = O.osk_unit(q, k, v, i, u["list"], u["k"], sh, opb)
    wg = O.osk_unit(q, k, v, i, u["list"], u["k"], sh, opg)
    assert wb["out"].shape == (rows, 128) and wg["out"].shape == (rows, 128)
    for g in range(4):
        if g * 32 < rows:
            assert np.array_equal(wg["status"][g], wb["status"])
        else:
            assert not wg["status"][g].any() and wg["groups"][g]["n_comp"] == 0
    assert np.allclose(wg["out"], wb["out"], atol=1e-12)
    # with skipping on, the group walks still give the closed form over their sets
    opm = O.OskParams(tight_budget=0.5, skip_mode=O.SKIP_MASS, vote_rows=32)
    wm = O.osk_unit(q, k, v, i, u["list"], u["k"], sh, opm)
    assert np.allclose(wm["out_walk"], wm["out"], atol=1e-12)


# ------------------------------------------------------------------ GQA-shared lists

def test_kv_group_lists_sum_per_head_contributions():
    # One list per KV head: S is the sum of the query heads' own block scores, the HRM
    # flags are the union of theirs, and with one query head per group the list is
    # that head's own.
    sh = _shape(seq_len=1024, block=64, head_dim=32, q_heads=3, kv_heads=1)
    qs = np.stack([_rand(1024, 32, 40 + h) for h in range(3)])
    k = _rand(1024, 32, 50)
    kp = O.KapParams(budget=0.3)
    shared = O.kap_kv_group(qs, k, sh, kp)
    per = [O.kap_head(qs[h], k, sh, kp) for h in range(3)]
    for i, u in enumerate(shared):
        assert np.allclose(u["S"], sum(p[i]["S"] for p in per), rtol=1e-12, atol=0)
        assert np.array_equal(u["hrm"], np.logical_or.reduce([p[i]["hrm"] for p in per]))
        assert u["k"] == per[0][i]["k"]
    one = O.kap_kv_group(qs[:1], k, sh, kp)
    for a, b in zip(one, per[0]):
        assert np.array_equal(a["list"], b["list"])


def test_kv_group_list_keeps_each_heads_planted_block():
    # Head 0 looks along u0, head 1 along u1; key block 2 is planted along u0 and key
    # block 5 along u1.  At a budget of two blocks, each head's own list leads with its
    # block, and the shared list holds both (each is some row's HRM block).
    rng = np.random.default_rng(3)
    n, d, B = 512, 32, 64
    u = np.linalg.qr(rng.standard_normal((d, 2)))[0].T.astype(np.float32)   # orthonormal
    k = 0.3 * rng.standard_normal((n, d)).astype(np.float32)
    k[2 * B:3 * B] += 12.0 * u[0]
    k[5 * B:6 * B] += 12.0 * u[1]
    qs = np.stack([0.3 * rng.standard_normal((n, d)).astype(np.float32) + 3.0 * u[h] for h in range(2)])
    sh = _shape(seq_len=n, block=B, head_dim=d, q_heads=2, kv_heads=1)
    kp = O.KapParams(budget=0.25)                          # n = 8 candidates at i = 7 -> k = 2
    i = 7
    own = [O.kap_head(qs[h], k, sh, kp, blocks=[i])[0] for h in range(2)]
    assert own[0]["list"][0] == 2 and own[1]["list"][0] == 5
    shared = O.kap_kv_group(qs, k, sh, kp, blocks=[i])[0]
    assert sorted(shared["list"].tolist()) == [2, 5]
    assert shared["hrm"][2] and shared["hrm"][5]


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_full_budget_is_dense(seed):
    # The first pin at random shapes: block 64 or 128, head dim 16 to 64, a ragged length of
    # 1 to 4 blocks, causal or not, the list visited in a random order; rho = rho' = 1 with
    # the skip test off is dense softmax attention (fp64 SDPA) for every query block.
    rng = np.random.default_rng(500 + seed)
    blk = int(rng.choice([64, 128]))
    d = int(rng.choice([16, 32, 64]))
    n = int(rng.integers(blk + 1, 4 * blk + 1))
    causal = bool(rng.random() < 0.5)
    sh = _shape(seq_len=n, block=blk, head_dim=d, causal=causal)
    q, k, v = (_rand(n, d, 600 + 3 * seed + s) for s in range(3))
    ref = _sdpa(q, k, v, causal)
    kp = O.KapParams(budget=1.0)
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF)
    for u, i in zip(O.kap_head(q, k, sh, kp), range(sh.nb)):
        assert sorted(u["list"]) == list(range(u["n"]))          # every candidate, once
        w = O.osk_unit(q, k, v, i, rng.permutation(u["list"]), u["k"], sh, op)
        rows = slice(i * blk, min(n, (i + 1) * blk))
        assert np.allclose(w["out"], ref[rows], atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(8))
def test_random_subsets_walk_order_invariance(seed):
    # Without skipping, the online-softmax result over any set of blocks does not depend on
    # the order they are visited in: random subsets of the candidates, random orders.
    rng = np.random.default_rng(700 + seed)
    blk, d, n = 64, 32, 1024
    sh = _shape(seq_len=n, block=blk, head_dim=d)
    q, k, v = (_rand(n, d, 800 + 3 * seed + s) for s in range(3))
    op = O.OskParams(tight_budget=1.0, skip_mode=O.SKIP_OFF)
    i = int(rng.integers(1, n // blk))
    lst = rng.choice(i + 1, size=int(rng.integers(1, i + 2)), replace=False)
    q_blk = q[i * blk:(i + 1) * blk]
    base = O.osk_walk(q_blk, k, v, i, lst, len(lst), sh, op)
    for _ in range(3):
        w = O.osk_walk(q_blk, k, v, i, rng.permutation(lst), len(lst), sh, op)
        assert np.allclose(w["out_walk"], base["out_walk"], atol=1e-12, rtol=0)
        assert np.allclose(w["lse_walk"], base["lse_walk"], atol=1e-12, rtol=0)
