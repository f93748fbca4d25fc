"""Tie-band comparator and decision replay (test infrastructure only).

Several results of the method are correct at once: blocks whose proxy scores
tie to within rounding may be ordered either way, and a skip decision whose
statistic sits on the threshold may go either way.  These helpers accept a
GPU result iff it is one of the results the oracle admits within a relative
band of 1e-5 on the deciding quantities, and they replay the oracle walk with
the GPU's decisions forced at such ambiguous positions.
"""
from __future__ import annotations

import numpy as np

TIE = 1e-5


def _hrm_bounds(P: np.ndarray, forced: np.ndarray, tie: float):
    """Per candidate: definitely HRM / possibly HRM under the tie band."""
    n = P.shape[1]
    definite = forced.copy()
    possible = forced.copy()
    for r in range(P.shape[0]):
        row = P[r]
        mx = row.max()
        near = np.nonzero(row >= mx - tie * max(1.0, abs(mx)))[0]
        possible[near] = True
        if near.size == 1:
            definite[near[0]] = True
    assert definite.shape == (n,)
    return definite, possible


def check_list(unit: dict, gpu_list, gpu_cnt: int, gpu_hrm_cnt: int,
               gpu_score=None, forced_hrm=None, tie: float = TIE):
    """Validate one GPU visit list against the oracle's KAP unit.

    Returns (ok, message).  unit is the dict returned by oracle.kap_unit.
    """
    n, k = unit["n"], unit["k"]
    S = unit["S"]
    gl = np.asarray(gpu_list, dtype=np.int64)
    klo, khi = unit.get("k_range", (k, k))
    if not (klo <= gpu_cnt <= khi):
        return False, f"count {gpu_cnt} outside [{klo}, {khi}]"
    k = gpu_cnt
    lst = gl[:k]
    if np.any(gl[k:] != -1):
        return False, "padding not -1"
    if np.any(lst < 0) or np.any(lst >= n):
        return False, f"index out of candidate range: {lst}"
    if len(set(lst.tolist())) != k:
        return False, "duplicate indices"
    if forced_hrm is None:
        forced_hrm = unit.get("forced")
    forced = np.zeros(n, dtype=bool) if forced_hrm is None else np.asarray(forced_hrm, dtype=bool)
    definite, possible = _hrm_bounds(unit["P"], forced, tie)
    if not (definite.sum() <= gpu_hrm_cnt <= possible.sum()):
        return False, f"hrm count {gpu_hrm_cnt} outside [{definite.sum()}, {possible.sum()}]"
    if unit.get("order_mode", 0) == 1:
        # plain top-k by S: one group; the HRM count is still checked above
        definite = np.zeros(n, dtype=bool)
        possible = np.zeros(n, dtype=bool)
        gpu_hrm_cnt = 0
    flag = np.arange(k) < min(gpu_hrm_cnt, k)
    for p, j in enumerate(lst):
        if flag[p] and not possible[j]:
            return False, f"position {p} block {j} flagged HRM, oracle says not"
        if not flag[p] and definite[j]:
            return False, f"position {p} block {j} not flagged HRM, oracle says HRM"

    def le(a, b):  # S[a] <= S[b] within the band
        return S[a] <= S[b] + tie * max(S[a], S[b])

    for p in range(k - 1):
        a, b = lst[p], lst[p + 1]
        if flag[p] == flag[p + 1] and not le(b, a):
            return False, f"order: S[{b}]={S[b]!r} after S[{a}]={S[a]!r}"
    excluded = np.setdiff1d(np.arange(n), lst)
    if excluded.size:
        last = lst[k - 1]
        if gpu_hrm_cnt >= k:
            # every listed block is HRM; excluded HRM blocks must not outrank the last one
            n_ex_hrm = gpu_hrm_cnt - k
            if not (definite[excluded].sum() <= n_ex_hrm <= possible[excluded].sum()):
                return False, "excluded HRM count inconsistent"
            for j in excluded:
                if definite[j] and not le(j, last):
                    return False, f"excluded HRM block {j} outranks listed {last}"
        else:
            for j in excluded:
                if definite[j]:
                    return False, f"excluded block {j} is HRM"
                if not le(j, last):
                    return False, f"excluded block {j} S={S[j]!r} > last listed {last} S={S[last]!r}"
    if gpu_score is not None:
        gs = np.asarray(gpu_score, dtype=np.float64)[:k]
        err = np.abs(gs - S[lst])
        if np.any(err > tie * np.maximum(1.0, S[lst])):
            return False, f"score mismatch, max err {err.max()}"
    return True, "ok"


def replay_walk(walk_fn, gpu_status, max_replays: int = 64):
    """Replay the oracle walk with the GPU's decisions forced at ambiguous positions.

    walk_fn(forced) -> dict from oracle.osk_walk / osk_unit.
    gpu_status: per-position status (0 not reached, 1 computed, 2 skipped).
    Returns (ok, walk, message, forced).
    """
    gs = np.asarray(gpu_status, dtype=np.int64)
    forced = {}
    w = None
    for _ in range(max_replays + 1):
        w = walk_fn(forced)
        os_ = w["status"][: gs.size]
        diff = np.nonzero(os_ != gs[: os_.size])[0]
        if diff.size == 0:
            if np.any(gs[os_.size:] != 0):
                return False, w, "gpu status beyond list", forced
            return True, w, "ok", forced
        p = int(diff[0])
        if gs[p] in (1, 2) and os_[p] in (1, 2) and p in w["margins"]:
            d, tol = w["margins"][p]
            if abs(d) <= tol:
                forced[p] = gs[p] == 2
                continue
            return False, w, f"decision at position {p}: gpu {gs[p]} oracle {os_[p]} margin {d} > tol {tol}", forced
        return False, w, f"status at position {p}: gpu {gs[p]} oracle {os_[p]}", forced
    return False, w, "too many replays", forced
