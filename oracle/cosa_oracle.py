"""fp64 CPU oracle of CoSA's prefill hot path: KAP (proxy) and OSK (kernel).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by the cpu_baseline leg of bench.py, never by the product path.  It shares no
code with the HIP library or its binding.

Sources (cited by page title and section; no formula, listing or constant is
printed on any of them, so every rule below is a reading of them, stated in the
docstring of the function that applies it):
  [Abstract]  authors' abstract of "CoSA: Accelerating Long-Context Inference
              via Proxy-Kernel Co-Designed Sparse Attention" (arXiv 2607.25291),
              as reproduced on insight.artgrammer.co.kr.
  [Summary]   gist.science (pt) "Resumo Técnico" of the same paper:
              §2.1 design principles, §2.2 Stage 1 KAP, §2.3 Stage 2 OSK.
  [TL;DR]     aitrending.vip article on the paper, "Technical Details".

Precision: everything is fp64 except the pooling step, which is defined
bitwise here (sequential fp32 sum, exact power-of-two scale, round to the
input dtype) so that pooled vectors are identical on every implementation.

Parity pins: see tests/test_oracle_pins.py.  Every function here is pinned
by at least one closed form, textbook special case or invariant; the only
unpinned items are the constants the pages never print (pool size g, skip
threshold eps, the aggregation rule), which are parameters.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# cap modes, skip modes, status codes
COMPUTED, VISITED = 0, 1
SKIP_OFF, SKIP_MAXDIFF, SKIP_MASS = 0, 1, 2
STATUS_NOT_REACHED, STATUS_COMPUTED, STATUS_SKIPPED = 0, 1, 2
POOL_MEAN, POOL_STRIDE = 0, 1
AGG_SUM, AGG_MAX = 0, 1
SEL_TOPK, SEL_CUMMASS = 0, 1
ORDER_HRM_FIRST, ORDER_SCORE = 0, 1


@dataclass
class Shape:
    batch: int
    q_heads: int
    kv_heads: int
    seq_len: int
    head_dim: int
    block: int
    causal: bool = True
    scale: float = 0.0          # 0 => 1/sqrt(head_dim)
    dtype: str = "bf16"         # "bf16" or "f32": storage dtype of Q, K, V, O

    @property
    def nb(self) -> int:
        """Key/query blocks; the last one is partial when block does not divide seq_len."""
        return -(-self.seq_len // self.block)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def n_cand(self, i: int) -> int:
        """Number of key blocks a query block may attend to."""
        return i + 1 if self.causal else self.nb


@dataclass
class KapParams:
    budget: float                 # rho in (0, 1]
    pool: int = 0                 # g, 0 => block // 4
    pool_mode: int = POOL_MEAN
    agg_mode: int = AGG_SUM
    sel_mode: int = SEL_TOPK
    mass: float = 0.9             # for SEL_CUMMASS
    force_sink: bool = False
    force_diag: bool = False
    order_mode: int = ORDER_HRM_FIRST   # ORDER_SCORE: by S alone (plain top-k proxy)

    def g(self, shape: Shape) -> int:
        return self.pool if self.pool > 0 else shape.block // 4


@dataclass
class OskParams:
    """Walk parameters.  cap_mode: the tightened budget caps the visited blocks (VISITED, the
    default reading: [Abstract] the kernel skips more blocks under a tightened budget, [Summary]
    §4 in-kernel skipping raises the sparsity) or the computed ones (COMPUTED)."""
    tight_budget: float           # rho' in (0, 1]
    cap_mode: int = VISITED
    skip_mode: int = SKIP_MASS
    skip_param: float = 1e-3      # MASS: eps; MAXDIFF: tau
    vote_rows: int = 0            # 0: the whole query block votes; r: each group of r rows


def budget_count(rho: float, n: int) -> int:
    """Blocks kept under a budget rho out of n candidates: min(n, max(1, ceil(rho*n))).

    The budget is a fraction of the candidate blocks of each query block
    ([Abstract]: a moderate budget for the proxy, a tightened one for the kernel;
    [Summary] §2.2, §2.3).
    The product is formed in IEEE double from the given values.
    """
    return int(min(n, max(1, math.ceil(float(rho) * float(n)))))


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage dtype, round-to-nearest-even."""
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


# ---------------------------------------------------------------- KAP stage

def pool_rows(x: np.ndarray, g: int, mode: int, dtype: str) -> np.ndarray:
    """Downsample rows of x [S, D] by g.  [Summary] §2.2, block ranking: the
    proxy downsamples queries and keys before scoring.

    MEAN: fp32 sum of the g rows in ascending order, times 2**-log2(g), then
    rounded to the storage dtype; a last, partial group sums only the rows that
    exist (same scale).  STRIDE: the first row of each group.
    Returns float32 [ceil(S/g), D] holding dtype-exact values.
    """
    s, d = x.shape
    assert g & (g - 1) == 0
    x = np.asarray(x, dtype=np.float32)
    full = s // g
    x3 = x[:full * g].reshape(full, g, d)
    if mode == POOL_STRIDE:
        return x[::g].copy()
    acc = x3[:, 0, :].copy()
    for t in range(1, g):
        acc = (acc + x3[:, t, :]).astype(np.float32)     # one fp32 rounding per add
    if s % g:
        tail = x[full * g:]
        last = tail[0].copy()
        for t in range(1, tail.shape[0]):
            last = (last + tail[t]).astype(np.float32)
        acc = np.concatenate([acc, last[None, :]])
    acc = (acc * np.float32(1.0 / g)).astype(np.float32)  # exact: power of two
    return round_to_dtype(acc, dtype)


def proxy_block_scores(qp: np.ndarray, kp: np.ndarray, i: int, shape: Shape,
                       g: int) -> np.ndarray:
    """Block-level proxy scores P[r, j] for the pooled rows r of query block i.

    [Summary] §2.2: approximate scores from the pooled vectors, then MaxPool
    over the keys of each block (keeping each row's maximum).
    P[r, j] = max over pooled keys t of block j visible from r of scale*q~_r.k~_t,
    with pooled key t visible from pooled query r iff t <= r (causal), and
    -inf where block j holds no visible pooled key.
    Returns fp64 [rows of block i (R_b, fewer in a partial last block), nb].
    """
    rb = shape.block // g
    nb = shape.nb
    npool = qp.shape[0]
    rows = np.arange(i * rb, min((i + 1) * rb, npool))    # the last block may hold fewer
    q = qp[rows].astype(np.float64)
    k = kp.astype(np.float64)
    s = shape.sm_scale * (q @ k.T)                         # [rows, N/g]
    if shape.causal:
        t = np.arange(k.shape[0])
        s[t[None, :] > rows[:, None]] = -np.inf
    pad = nb * rb - s.shape[1]                             # pooled keys past the sequence
    if pad:
        s = np.concatenate([s, np.full((s.shape[0], pad), -np.inf)], axis=1)
    return s.reshape(len(rows), nb, rb).max(axis=2)


def kap_unit(P: np.ndarray, i: int, shape: Shape, kp_: KapParams) -> dict:
    """Order and select the key blocks of query block i from its proxy scores.

    [Summary] §2.2: MaxNorm turns each row's block scores into relative
    contributions; blocks holding some row's maximum are flagged HRM; the
    computation-order mask visits HRM blocks first, then the rest by
    estimated score.  [Abstract]: the proxy keeps blocks under a moderate
    budget and the order it emits is the order the kernel visits KV pages.
    """
    n = shape.n_cand(i)
    cand = np.arange(n)
    Pc = P[:, :n]
    rowmax = Pc.max(axis=1)
    c = np.exp(Pc - rowmax[:, None])                       # MaxNorm: in (0, 1], one 1 per row
    if kp_.agg_mode == AGG_SUM:
        S = c.sum(axis=0)
    else:
        S = c.max(axis=0)
    hrm = np.zeros(n, dtype=bool)
    hrm[np.argmax(Pc, axis=1)] = True                      # lowest j wins exact ties
    forced = np.zeros(n, dtype=bool)
    if kp_.force_sink:
        forced[0] = True
    if kp_.force_diag:
        forced[min(i, n - 1)] = True
    hrm |= forced
    first = hrm if kp_.order_mode == ORDER_HRM_FIRST else np.zeros(n, dtype=bool)
    order = np.lexsort((cand, -S, -first.astype(np.int64)))  # HRM desc, S desc, j asc
    k = budget_count(kp_.budget, n)
    k_range = (k, k)
    if kp_.sel_mode == SEL_CUMMASS:
        # the shortest prefix of the visiting order whose score sum reaches mass * total,
        # at least 1 and at most k blocks
        total = S.sum()
        goal = kp_.mass * total
        cum = np.cumsum(S[order])
        hit = np.nonzero(cum >= goal)[0]
        klen = int(hit[0]) + 1 if hit.size else n
        ktop = k
        k = max(1, min(ktop, klen))
        # lengths a correct implementation may return when a prefix sum sits within the
        # relative band of the goal (rounding of the sums)
        band = 1e-5 * goal
        ok = [L for L in range(1, ktop + 1)
              if (cum[L - 1] >= goal - band or L == ktop) and (L == 1 or cum[L - 2] < goal + band)]
        k_range = (min(ok), max(ok))
    sel = order[:k]
    return dict(list=sel.astype(np.int64), hrm=hrm, forced=forced, S=S, P=Pc, rowmax=rowmax,
                hrm_cnt=int(hrm.sum()), score=S[sel], k=k, k_range=k_range, n=n,
                order_mode=kp_.order_mode)


def kap_head(q_head: np.ndarray, k_head: np.ndarray, shape: Shape,
             kp_: KapParams, blocks=None) -> list:
    """KAP for one query head against its KV head.  q_head, k_head: [N, D]."""
    g = kp_.g(shape)
    qp = pool_rows(q_head, g, kp_.pool_mode, shape.dtype)
    kp = pool_rows(k_head, g, kp_.pool_mode, shape.dtype)
    out = []
    for i in (range(shape.nb) if blocks is None else blocks):
        P = proxy_block_scores(qp, kp, i, shape, g)
        out.append(kap_unit(P, i, shape, kp_))
    return out


def kap_kv_group(q_heads, k_head: np.ndarray, shape: Shape, kp_: KapParams, blocks=None) -> list:
    """KAP with one list per KV head, shared by its query heads (GQA).

    The pages rank blocks per query head.  This mode takes the plainest
    extension to a shared list: the pooled rows of all query heads of the group
    (heads in ascending order) are the rows of the query block, so every row
    contributes its MaxNorm values to S and its HRM block to the flags, and the
    order and budget are those of a single unit.  q_heads: [G, N, D].
    """
    g = kp_.g(shape)
    kp = pool_rows(k_head, g, kp_.pool_mode, shape.dtype)
    qps = [pool_rows(qh, g, kp_.pool_mode, shape.dtype) for qh in q_heads]
    out = []
    for i in (range(shape.nb) if blocks is None else blocks):
        P = np.concatenate([proxy_block_scores(qp, kp, i, shape, g) for qp in qps], axis=0)
        out.append(kap_unit(P, i, shape, kp_))
    return out


# ---------------------------------------------------------------- OSK stage

def _tile_scores(q_blk, k_blk, i, j, shape, row0=0):
    """Logits of query rows row0 .. row0 + len(q_blk) - 1 of block i against block j."""
    s = shape.sm_scale * (q_blk @ k_blk.T)                 # [rows, keys of block j]
    if shape.causal and j == i:
        r = row0 + np.arange(q_blk.shape[0])
        c = np.arange(k_blk.shape[0])
        s[c[None, :] > r[:, None]] = -np.inf               # key c > query r masked
    return s


def osk_walk(q_blk: np.ndarray, k_head: np.ndarray, v_head: np.ndarray, i: int,
             visit: np.ndarray, k_kap: int, shape: Shape, op: OskParams,
             page_table=None, forced=None, row0: int = 0) -> dict:
    """Walk the ordered list of query block i with online softmax and skipping.

    [Summary] §2.3: blocks outside the list are never touched (mask-skipped);
    for listed blocks the kernel compares the block's local max with the
    running online-softmax statistics and skips it when negligible
    (in-kernel skipped); the rest are computed.  [Abstract]: the kernel skips
    more blocks under a tightened budget.  [Summary] §2.1: the accumulation
    does not depend on the visiting order.

    visit: list of logical key-block indices (length >= k_kap; first k_kap used).
    forced: optional {position: skip?} overriding the skip test (replay).
    q_blk may be a group of rows of the block starting at row row0 (per-group vote).
    Returns the status of each position, the computed blocks in visit order,
    the walk's own output acc/l, its LSE, and for each tested position the
    decision margin max_r(stat_r - thr) with its tolerance.
    """
    rows = q_blk.shape[0]
    B = shape.block
    n = shape.n_cand(i)
    kprime = min(k_kap, budget_count(op.tight_budget, n))
    if rows == 0:
        # a row group wholly past the end of the sequence takes no part
        return dict(status=np.zeros(len(visit), dtype=np.int64), computed=np.zeros(0, np.int64),
                    out_walk=np.zeros((0, q_blk.shape[1])), lse_walk=np.zeros(0),
                    n_comp=0, visited=0, kprime=kprime, margins={})
    q = q_blk.astype(np.float64)
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    acc = np.zeros((rows, q.shape[1]))
    n_comp = 0
    status = np.zeros(len(visit), dtype=np.int64)
    margins = {}
    computed = []
    visited = 0
    for p in range(k_kap):
        if op.cap_mode == COMPUTED and n_comp == kprime:
            break
        if op.cap_mode == VISITED and p == kprime:
            break
        j = int(visit[p])
        phys = j if page_table is None else int(page_table[j])
        kb = k_head[phys * B:(phys + 1) * B].astype(np.float64)
        vb = v_head[phys * B:(phys + 1) * B].astype(np.float64)
        s = _tile_scores(q, kb, i, j, shape, row0)
        visited += 1
        m_loc = s.max(axis=1)
        skip = False
        if n_comp > 0 and op.skip_mode != SKIP_OFF:
            if op.skip_mode == SKIP_MAXDIFF:
                stat = m_loc - m
                thr = op.skip_param
            else:
                nv = np.isfinite(s).sum(axis=1)
                stat = m_loc - m + np.log(nv) - np.log(l)
                thr = math.log(op.skip_param)
            d = stat - thr
            r = int(np.argmax(d))
            tol = 1e-5 * max(1.0, abs(m[r]), abs(m_loc[r]))
            margins[p] = (float(d[r]), tol)
            skip = bool(np.all(d <= 0.0))
            if forced is not None and p in forced:
                skip = bool(forced[p])
        if skip:
            status[p] = STATUS_SKIPPED
            continue
        m_new = np.maximum(m, m_loc)
        alpha = np.exp(m - m_new)                          # exp(-inf) = 0 on the first block
        P = np.exp(s - m_new[:, None])
        l = alpha * l + P.sum(axis=1)
        acc = alpha[:, None] * acc + P @ vb
        m = m_new
        status[p] = STATUS_COMPUTED
        computed.append(j)
        n_comp += 1
    return dict(status=status, computed=np.array(computed, dtype=np.int64),
                out_walk=acc / l[:, None], lse_walk=m + np.log(l),
                n_comp=n_comp, visited=visited, kprime=kprime, margins=margins)


def restricted_attention(q_blk, k_head, v_head, i, blocks, shape: Shape,
                         page_table=None, row0=0):
    """Closed form of the OSK output for query block i given its computed blocks C:
    O[q] = sum_{c in V_q} e^{s_qc} v_c / sum_{c in V_q} e^{s_qc}, where V_q are
    the keys of C visible from q (keys past the end of the sequence do not
    exist).  Returns (O [rows, D] fp64, LSE [rows] fp64).
    """
    B = shape.block
    q = q_blk.astype(np.float64)
    ss, vs = [], []
    for j in blocks:
        phys = int(j) if page_table is None else int(page_table[int(j)])
        ss.append(_tile_scores(q, k_head[phys * B:(phys + 1) * B].astype(np.float64), i, int(j), shape, row0))
        vs.append(v_head[phys * B:(phys + 1) * B].astype(np.float64))
    s = np.concatenate(ss, axis=1)
    v = np.concatenate(vs, axis=0)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1)
    return (e @ v) / den[:, None], mx[:, 0] + np.log(den)


def osk_unit(q_head, k_head, v_head, i, visit, k_kap, shape, op, page_table=None,
             forced=None, group=None) -> dict:
    """OSK for one query block: walk for the decisions, closed form for the output.

    With op.vote_rows = r < B every group of r rows walks the list on its own (its own
    skip votes, cap and status); group selects one of them (rows g*r .. g*r + r - 1).
    """
    B = shape.block
    r = op.vote_rows if 0 < op.vote_rows < B else B
    if group is None and r < B:
        # all groups: statuses stacked per group, outputs concatenated along the rows
        ws = [osk_unit(q_head, k_head, v_head, i, visit, k_kap, shape, op, page_table, forced, g)
              for g in range(B // r)]
        return dict(status=np.stack([w["status"] for w in ws]),
                    computed=[w["computed"] for w in ws],
                    out=np.concatenate([w["out"] for w in ws]),
                    lse=np.concatenate([w["lse"] for w in ws]),
                    out_walk=np.concatenate([w["out_walk"] for w in ws]),
                    lse_walk=np.concatenate([w["lse_walk"] for w in ws]),
                    n_comp=sum(w["n_comp"] for w in ws), visited=max(w["visited"] for w in ws),
                    kprime=ws[0]["kprime"], groups=ws)
    g = 0 if group is None else group
    q_blk = q_head[i * B + g * r:i * B + (g + 1) * r]
    w = osk_walk(q_blk, k_head, v_head, i, visit, k_kap, shape, op, page_table, forced, g * r)
    if q_blk.shape[0] == 0:
        w["out"], w["lse"] = w["out_walk"], w["lse_walk"]
        return w
    o, lse = restricted_attention(q_blk, k_head, v_head, i, w["computed"], shape, page_table, g * r)
    w["out"] = o
    w["lse"] = lse
    return w


def run_head(q_head, k_head, v_head, shape: Shape, kp_: KapParams, op: OskParams,
             blocks=None) -> list:
    """KAP then OSK for every (or the given) query block of one head."""
    units = kap_head(q_head, k_head, shape, kp_, blocks)
    res = []
    for u, i in zip(units, range(shape.nb) if blocks is None else blocks):
        w = osk_unit(q_head, k_head, v_head, i, u["list"], u["k"], shape, op)
        res.append(dict(kap=u, osk=w, i=i))
    return res


def dense_attention(q_head, k_head, v_head, shape: Shape):
    """Textbook softmax attention (causal if shape.causal) of one head, fp64.

    The sparse method is measured against it ([Abstract]; [Summary] §4,
    efficiency) and reduces to it at full budget with skipping off.
    Returns (O [N, D], LSE [N]).
    """
    q = q_head.astype(np.float64)
    k = k_head.astype(np.float64)
    v = v_head.astype(np.float64)
    s = shape.sm_scale * (q @ k.T)
    if shape.causal:
        n = s.shape[0]
        idx = np.arange(n)
        s[idx[None, :] > idx[:, None]] = -np.inf
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1)
    return (e @ v) / den[:, None], mx[:, 0] + np.log(den)
