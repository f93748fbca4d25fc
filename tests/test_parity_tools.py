"""CPU tests of the parity machinery the full-size GPU tests use: the output criterion
(tests/oracle_pool.output_check) and the per-head checker the worker pool runs.  The checker is
fed the oracle's own results (it must accept them) and results with planted mistakes (it must
reject each)."""
import numpy as np

import oracle as O
from oracle_pool import TOL_LSE, _bf16_neighbours, check_head, output_check
from synth import config, make, shrink


def test_bf16_neighbours():
    x = np.array([1.0, -1.0, 0.0, 3.0], np.float32)
    down, up = _bf16_neighbours(x)
    assert down.tolist() == [1 - 2 ** -8, -(1 + 2 ** -7), -(2.0 ** -133), 3 - 2 ** -6]
    assert up.tolist() == [1 + 2 ** -7, -(1 - 2 ** -8), 2.0 ** -133, 3 + 2 ** -6]


def test_output_check_is_rounding_of_a_value_within_tolerance():
    # bf16 at 1.0: one ulp up is 1 + 2^-7; its rounding interval [1 + 2^-8, 1 + 3 * 2^-8] meets
    # [0.99, 1.01]; two ulps up ([1 + 3 * 2^-8, 1 + 5 * 2^-8]) does not
    ref = np.array([1.0])
    assert output_check(np.array([1 + 2 ** -7], np.float32), ref, "bf16")[0] <= 0
    e = output_check(np.array([1 + 2 ** -6], np.float32), ref, "bf16")[0]
    assert abs(e - (1 + 3 * 2 ** -8 - 1.01)) < 1e-12
    # at 4.0 (ulp 2^-5) the stored value nearest to 4.0 passes for ref = 4.0 + 0.0249; 4 + 2^-5 too
    ref = np.array([4.0249])
    assert output_check(np.array([4.0], np.float32), ref, "bf16")[0] <= 0
    assert output_check(np.array([4.0 + 2 ** -5], np.float32), ref, "bf16")[0] <= 0
    assert output_check(np.array([4.0 - 2 ** -5], np.float32), ref, "bf16")[0] > 0
    # fp32: tolerance 1e-4
    ref = np.array([1.0])
    assert output_check(np.array([1.00009], np.float32), ref, "f32")[0] <= 0
    assert output_check(np.array([1.00011], np.float32), ref, "f32")[0] > 0
    # the flat measures
    _, flat, flat_r, n, nr = output_check(np.array([1 + 2 ** -7, 0.5], np.float32),
                                          np.array([1.001, 0.5]), "bf16")
    assert abs(flat - (1 + 2 ** -7 - 1.001)) < 1e-12 and flat_r == 2 ** -7 and n == 0 and nr == 0


def _oracle_job(cfg, h=0):
    x = make(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    B, N = cfg["block"], cfg["seq_len"]
    sh = O.Shape(1, cfg["q_heads"], cfg["kv_heads"], N, cfg["head_dim"], B, True,
                 float(np.float32(1.0 / np.sqrt(cfg["head_dim"]))), cfg["dtype"])
    kp = O.KapParams(budget=cfg["budget"])
    op = O.OskParams(tight_budget=cfg["tight_budget"])
    units = O.kap_head(x["q"][0, h], x["k"][0, h // G], sh, kp)
    nb = len(units)
    kmax = max(u["k"] for u in units)
    idx = np.full((nb, kmax), -1, np.int32)
    sc = np.zeros((nb, kmax), np.float32)
    cnt = np.zeros(nb, np.int32)
    hrm = np.zeros(nb, np.int32)
    st = np.zeros((nb, kmax), np.uint8)
    tc = np.zeros((nb, 2), np.int32)
    out = np.zeros((N, cfg["head_dim"]), np.float32)
    lse = np.zeros(N, np.float32)
    for i, u in enumerate(units):
        idx[i, :u["k"]] = u["list"]
        sc[i, :u["k"]] = u["score"]
        cnt[i], hrm[i] = u["k"], u["hrm_cnt"]
        w = O.osk_unit(x["q"][0, h], x["k"][0, h // G], x["v"][0, h // G], i, u["list"], u["k"],
                       sh, op)
        st[i, :u["k"]] = w["status"][:u["k"]]
        tc[i] = (w["visited"], w["n_comp"])
        out[i * B:(i + 1) * B] = O.round_to_dtype(w["out"].astype(np.float32), cfg["dtype"])
        lse[i * B:(i + 1) * B] = w["lse"]
    bits = (out.view(np.uint32) >> 16).astype(np.uint16)
    return dict(cfg=cfg, kap=dict(budget=kp.budget), osk=dict(tight_budget=op.tight_budget),
                b=0, h=h, share=False, idx=idx, cnt=cnt, hrm=hrm, sc=sc, st=st, tc=tc, out=bits,
                lse=lse)


def test_head_checker_accepts_the_oracle_and_rejects_planted_mistakes():
    cfg = shrink(config(1), 2048, q_heads=2, kv_heads=1, n_salient=3)
    cfg.update(salient_gain=12.0, q_noise=0.2, budget=0.6, tight_budget=0.6)   # skips fire
    job = _oracle_job(cfg, h=1)
    r = check_head(job)
    assert r["n_bad"] == 0 and r["excess"] <= 0 and r["units"] == 16, r
    assert r["skipped"] > 0
    # each mistake is planted alone and must be reported by its own check
    def rejected(r, kind):
        return r["n_bad"] >= 1 and any(m.startswith(kind) for m in r["bad"])
    # a list out of order (the first and last of a long list swapped)
    bad = dict(job, idx=job["idx"].copy())
    i = 15
    k = int(job["cnt"][i])
    bad["idx"][i, [0, k - 1]] = bad["idx"][i, [k - 1, 0]]
    assert rejected(check_head(bad), "list")
    # a skip decision flipped far from the threshold, the tile counts made to agree with it
    bad = dict(job, st=job["st"].copy(), tc=job["tc"].copy())
    i, p = [(i, p) for i in range(16) for p in range(int(job["cnt"][i])) if job["st"][i, p] == 2][0]
    bad["st"][i, p] = 1
    bad["tc"][i, 1] += 1
    assert rejected(check_head(bad), "walk")
    # an output off by 0.02
    bad = dict(job, out=job["out"].copy())
    f = (bad["out"][200:201].astype(np.uint32) << 16).view(np.float32) + np.float32(0.02)
    bad["out"][200:201] = (f.view(np.uint32) >> 16).astype(np.uint16)
    r = check_head(bad)
    assert r["excess"] > 0 and r["n_bad"] == 0
    # an LSE off by 2e-3 (twice the bf16 tolerance)
    bad = dict(job, lse=job["lse"].copy())
    bad["lse"][300] += np.float32(2e-3)
    r = check_head(bad)
    assert r["lse"] > TOL_LSE["bf16"] and r["excess"] <= 0
    # wrong tile counts: computed, then visited
    for c in (1, 0):
        bad = dict(job, tc=job["tc"].copy())
        bad["tc"][3, c] += 1
        assert rejected(check_head(bad), "counts")


def test_head_checker_block_ranges_cover_the_head():
    """A head cut into ranges of query blocks (the rows of out and lse sliced to each range) is
    checked unit for unit as the whole head is; a planted mistake is found in its range."""
    cfg = shrink(config(1), 2048, q_heads=2, kv_heads=1, n_salient=3)
    cfg.update(salient_gain=12.0, q_noise=0.2, budget=0.6, tight_budget=0.6)
    job = _oracle_job(cfg, h=0)
    B = cfg["block"]
    whole = check_head(job)
    parts = []
    for lo, hi in ((0, 5), (5, 11), (11, 16)):
        rows = slice(lo * B, hi * B)
        parts.append(check_head(dict(job, blocks=(lo, hi), out=job["out"][rows], lse=job["lse"][rows])))
    assert sum(p["units"] for p in parts) == whole["units"] == 16
    assert sum(p["skipped"] for p in parts) == whole["skipped"]
    assert max(p["excess"] for p in parts) == whole["excess"]
    assert all(p["n_bad"] == 0 for p in parts)
    bad = dict(job, out=job["out"].copy())
    f = (bad["out"][12 * B + 3:12 * B + 4].astype(np.uint32) << 16).view(np.float32) + np.float32(0.05)
    bad["out"][12 * B + 3:12 * B + 4] = (f.view(np.uint32) >> 16).astype(np.uint16)
    rows = slice(11 * B, 16 * B)
    assert check_head(dict(bad, blocks=(11, 16), out=bad["out"][rows], lse=bad["lse"][rows]))["excess"] > 0
    rows = slice(0, 11 * B)
    assert check_head(dict(bad, blocks=(0, 11), out=bad["out"][rows], lse=bad["lse"][rows]))["excess"] <= 0


def test_out_excess_applies_both_bounds():
    # The GPU tests' criterion: the rounding interval of the stored value must meet the
    # tolerance band AND |got - ref| <= 1e-2 + 2^-9 |ref| (bf16).  At ref = 4.0249 the stored
    # 4.0 passes the first (its interval reaches 4 + 2^-6) but misses the second by
    # 0.0249 - (0.01 + 4.0249 / 512) = 0.00704; at ref = 4.012 it passes both.
    import gpu_helpers
    saved = dict(gpu_helpers.FLAT_STATS)      # (the session's GPU error totals stay untouched)
    try:
        e = gpu_helpers.out_excess(np.array([4.0], np.float32), np.array([4.0249]), "bf16")
        assert abs(e - (0.0249 - 0.01 - 4.0249 / 512)) < 1e-9
        assert gpu_helpers.out_excess(np.array([4.0], np.float32), np.array([4.012]), "bf16") <= 0
        # and an output whose interval misses the band fails however the flat bound reads
        assert gpu_helpers.out_excess(np.array([1 + 2 ** -6], np.float32), np.array([1.0]), "bf16") > 0
        assert gpu_helpers.out_excess(np.array([1.00011], np.float32), np.array([1.0]), "f32") > 0
    finally:
        gpu_helpers.FLAT_STATS.clear()
        gpu_helpers.FLAT_STATS.update(saved)
