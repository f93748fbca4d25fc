"""CoSA block-sparse prefill attention for MI355X (gfx950): Python binding.

Thin ctypes layer over libcosa.so.  It only marshals arguments: torch provides
device memory and the current HIP stream, every step of the computation runs in
the library's HIP kernels.  There is no CPU fallback: if the library is missing
the import of the binding functions raises.

    idx, cnt, hrm = kap(q, k, block=128, budget=0.1)
    out = osk(q, k, v, idx, cnt, block=128, tight_budget=0.05)
    ref = dense(q, k, v, block=128)
"""
from __future__ import annotations

import ctypes

from ._lib import (  # noqa: F401
    COSA_BF16, COSA_F32, CAP_COMPUTED, CAP_VISITED, SKIP_MAXDIFF, SKIP_MASS, SKIP_OFF,
    KapParams, OskParams, Shape, CosaError, lib, lib_path, check,
)

__all__ = ["kap", "kap_noalloc", "osk", "prefill", "Pipeline", "dense", "list_capacity", "kap_workspace_bytes", "make_shape",
           "KapParams", "OskParams", "Shape", "CosaError", "lib", "lib_path"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return COSA_BF16
    if t.dtype == torch.float32:
        return COSA_F32
    raise CosaError(-2, f"unsupported dtype {t.dtype}")


def make_shape(q, k, block: int, causal: bool = True, scale: float = 0.0, seq_lens=None) -> Shape:
    """Shape of q [batch, q_heads, seq, dim] and k [batch, kv_heads, seq, dim].

    seq_lens: optional per-entry token counts (a varlen batch in a padded layout).
    """
    if q.dim() != 4 or k.dim() != 4:
        raise CosaError(-1, "q and k must be [batch, heads, seq, dim]")
    bt, hq, n, d = q.shape
    sh = Shape(bt, hq, k.shape[1], n, d, block, 1 if causal else 0, float(scale), _dtype_code(q))
    if seq_lens is not None:
        lens = [int(x) for x in seq_lens]
        if len(lens) != bt:
            raise CosaError(-1, f"seq_lens has {len(lens)} entries, expected {bt}")
        arr = (ctypes.c_int32 * bt)(*lens)
        sh._lens = arr                      # keeps the host array alive with the shape
        sh.seq_lens = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return sh


def _check_tensor(t, name, shape=None, dtype=None, device=None):
    if not t.is_cuda:
        raise CosaError(-1, f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise CosaError(-1, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise CosaError(-1, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise CosaError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise CosaError(-1, f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_qkv(q, k, v=None):
    """q [batch, q_heads, seq, dim]; k (and v) [batch, kv_heads, seq, dim] of q's dtype, on q's
    device.  The library takes every size but the KV head count from q, so a k or v with
    other sizes would be read past its end: this is checked before any call."""
    _check_tensor(q, "q")
    if q.dim() != 4:
        raise CosaError(-1, "q must be [batch, heads, seq, dim]")
    bt, _, n, d = q.shape
    if k.dim() != 4:
        raise CosaError(-1, "k must be [batch, heads, seq, dim]")
    _check_tensor(k, "k", shape=(bt, k.shape[1], n, d), dtype=q.dtype, device=q.device)
    if v is not None:
        _check_tensor(v, "v", shape=k.shape, dtype=q.dtype, device=q.device)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def list_capacity(shape: Shape, budget: float) -> int:
    r = lib().cosa_list_capacity(ctypes.byref(shape), ctypes.c_double(budget))
    check(r)
    return r


def kap_workspace_bytes(shape: Shape, params: KapParams) -> int:
    n = lib().cosa_kap_workspace_bytes(ctypes.byref(shape), ctypes.byref(params))
    if n == 0:
        raise CosaError(-1, "invalid shape or proxy parameters")
    return n


def kap(q, k, block: int, budget: float, pool: int = 0, pool_mode: int = 0, agg_mode: int = 0,
        force_sink: bool = False, force_diag: bool = False, causal: bool = True,
        scale: float = 0.0, kmax: int | None = None, return_scores: bool = False,
        workspace=None, outs=None, sel_mode: int = 0, mass: float = 0.9, order_mode: int = 0,
        seq_lens=None, share_kv: bool = False, stream=None):
    """Kernel-Aware Proxy: ordered per-query-block visit lists.

    Returns (visit_idx [B,H,nb,kmax] int32, visit_cnt [B,H,nb] int32,
    hrm_cnt [B,H,nb] int32[, visit_score [B,H,nb,kmax] float32]) with H the query
    heads, or the KV heads with share_kv (one list per KV head).
    """
    torch = _torch()
    shape = make_shape(q, k, block, causal, scale, seq_lens)
    params = KapParams(float(budget), int(pool), int(pool_mode), int(agg_mode), int(sel_mode),
                       float(mass), int(force_sink), int(force_diag), int(order_mode), int(share_kv))
    _check_qkv(q, k)
    dev = q.device
    nb = -(-shape.seq_len // block) if block > 0 else 0     # last block may be partial
    cap = list_capacity(shape, budget)
    kmax = cap if kmax is None else int(kmax)
    noalloc = workspace is _NOALLOC
    if not noalloc:
        wsb = kap_workspace_bytes(shape, params)
        if workspace is None:
            workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
        _check_tensor(workspace, "workspace", dtype=torch.uint8, device=dev)
    bt, hq = shape.batch, (shape.kv_heads if share_kv else shape.q_heads)
    if outs is not None:
        idx, cnt, hrm = outs[:3]
        sc = outs[3] if return_scores else None
        _check_tensor(idx, "visit_idx", shape=(bt, hq, nb, kmax), dtype=torch.int32, device=dev)
        _check_tensor(cnt, "visit_cnt", shape=(bt, hq, nb), dtype=torch.int32, device=dev)
        _check_tensor(hrm, "hrm_cnt", shape=(bt, hq, nb), dtype=torch.int32, device=dev)
        if sc is not None:
            _check_tensor(sc, "visit_score", shape=(bt, hq, nb, kmax), dtype=torch.float32,
                          device=dev)
    else:
        idx = torch.empty((bt, hq, nb, kmax), dtype=torch.int32, device=q.device)
        cnt = torch.empty((bt, hq, nb), dtype=torch.int32, device=q.device)
        hrm = torch.empty((bt, hq, nb), dtype=torch.int32, device=q.device)
        sc = torch.empty((bt, hq, nb, kmax), dtype=torch.float32, device=q.device) if return_scores else None
    if noalloc:
        r = lib().cosa_proxy_select_noalloc(ctypes.byref(shape), ctypes.byref(params), _ptr(q),
                                            _ptr(k), _ptr(idx), _ptr(cnt), _ptr(hrm), _ptr(sc),
                                            ctypes.c_int(kmax), _stream(stream))
    else:
        r = lib().cosa_proxy_select(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k),
                                    _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                    _ptr(idx), _ptr(cnt), _ptr(hrm), _ptr(sc), ctypes.c_int(kmax),
                                    _stream(stream))
    check(r)
    return (idx, cnt, hrm, sc) if return_scores else (idx, cnt, hrm)


_NOALLOC = object()   # the workspace marker that selects cosa_proxy_select_noalloc


def kap_noalloc(q, k, block: int, budget: float, **kw):
    """kap() through cosa_proxy_select_noalloc: the library's static device scratch serves as
    the workspace (no workspace is allocated or passed; outputs as kap's, allocated here unless
    `outs` gives them).  Calls overlapping on one GPU race on that scratch."""
    if "workspace" in kw:
        raise CosaError(-1, "kap_noalloc takes no workspace")
    return kap(q, k, block, budget, workspace=_NOALLOC, **kw)


def osk(q, k, v, visit_idx, visit_cnt, block: int, tight_budget: float,
        cap_mode: int = CAP_VISITED, skip_mode: int = SKIP_MASS, skip_param: float = 1e-3,
        page_table=None, causal: bool = True, scale: float = 0.0, return_lse: bool = False,
        return_status: bool = False, return_counts: bool = False, out=None, vote_rows: int = 0,
        seq_lens=None, shared_lists: bool = False, stream=None):
    """Ordered-Skipping Kernel.  Returns out (and, as asked, lse, status, counts)."""
    torch = _torch()
    shape = make_shape(q, k, block, causal, scale, seq_lens)
    params = OskParams(float(tight_budget), int(cap_mode), int(skip_mode), float(skip_param),
                       int(vote_rows), int(shared_lists))
    _check_qkv(q, k, v)
    dev = q.device
    bt, hq, n, d = q.shape
    nb = -(-n // block) if block > 0 else 0
    _check_tensor(visit_idx, "visit_idx", dtype=torch.int32, device=dev)
    hl = k.shape[1] if shared_lists else hq               # heads the lists are indexed by
    if visit_idx.dim() != 4 or tuple(visit_idx.shape[:3]) != (bt, hl, nb):
        raise CosaError(-1, f"visit_idx must be [batch, {'kv' if shared_lists else 'q'}_heads, nb, kmax]")
    kmax = visit_idx.shape[3]
    _check_tensor(visit_cnt, "visit_cnt", shape=(bt, hl, nb), dtype=torch.int32, device=dev)
    if page_table is not None:
        _check_tensor(page_table, "page_table", shape=(bt, nb), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", shape=q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty((bt, hq, n), dtype=torch.float32, device=q.device) if return_lse else None
    st = torch.empty((bt, hq, nb, kmax), dtype=torch.uint8, device=q.device) if return_status else None
    tc = torch.empty((bt, hq, nb, 2), dtype=torch.int32, device=q.device) if return_counts else None
    r = lib().cosa_ordered_sparse_attn(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(visit_idx), _ptr(visit_cnt), ctypes.c_int(kmax),
                                       _ptr(page_table), _ptr(out), _ptr(lse), _ptr(st), _ptr(tc),
                                       _stream(stream))
    check(r)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_status:
        res.append(st)
    if return_counts:
        res.append(tc)
    return res[0] if len(res) == 1 else tuple(res)


class Pipeline:
    """The two streams and the event cosa_prefill pipelines over (default priority streams)."""

    def __init__(self, device=None):
        torch = _torch()
        self.proxy = torch.cuda.Stream(device=device)
        self.walk = torch.cuda.Stream(device=device)
        self.event = torch.cuda.Event()
        self.event.record(self.walk)          # creates the underlying event
        self.walk.synchronize()


_PIPELINES = {}


def prefill(q, k, v, block: int, budget: float, tight_budget: float, head_chunks: int = 0,
            pool: int = 0, pool_mode: int = 0, agg_mode: int = 0, sel_mode: int = 0,
            mass: float = 0.9, force_sink: bool = False, force_diag: bool = False,
            order_mode: int = 0, share_kv: bool = False, cap_mode: int = CAP_VISITED,
            skip_mode: int = SKIP_MASS, skip_param: float = 1e-3, vote_rows: int = 0,
            causal: bool = True, scale: float = 0.0, seq_lens=None,
            return_lse: bool = False, return_lists: bool = False, out=None, workspace=None,
            lists=None, pipeline: Pipeline | None = None):
    """Proxy then walk over one layer, pipelined over groups of KV heads on two streams
    (cosa_prefill).  head_chunks 0 picks four groups (or the largest divisor of kv_heads below
    four) for sequences of 64K tokens and more, and one group below: shorter layers lose more to
    the extra launches and walk tails than the overlap saves.  The two streams wait for the
    current stream first, and the current stream waits for the walk at the end.  Returns out
    (and lse, and (visit_idx, visit_cnt, hrm_cnt) as asked)."""
    torch = _torch()
    shape = make_shape(q, k, block, causal, scale, seq_lens)
    kparams = KapParams(float(budget), int(pool), int(pool_mode), int(agg_mode), int(sel_mode),
                        float(mass), int(force_sink), int(force_diag), int(order_mode), int(share_kv))
    oparams = OskParams(float(tight_budget), int(cap_mode), int(skip_mode), float(skip_param),
                        int(vote_rows), int(share_kv))
    _check_qkv(q, k, v)
    dev = q.device
    bt, hq, n, d = q.shape
    hkv = k.shape[1]
    if head_chunks == 0:
        head_chunks = max(c for c in (1, 2, 4) if hkv % c == 0) if n >= 65536 else 1
    nb = -(-n // block) if block > 0 else 0
    kmax = list_capacity(shape, budget)
    if workspace is None:
        workspace = torch.empty(kap_workspace_bytes(shape, kparams), dtype=torch.uint8, device=q.device)
    hl = hkv if share_kv else hq
    if lists is None:
        lists = (torch.empty((bt, hl, nb, kmax), dtype=torch.int32, device=q.device),
                 torch.empty((bt, hl, nb), dtype=torch.int32, device=q.device),
                 torch.empty((bt, hl, nb), dtype=torch.int32, device=q.device))
    idx, cnt, hrm = lists
    _check_tensor(workspace, "workspace", dtype=torch.uint8, device=dev)
    _check_tensor(idx, "visit_idx", shape=(bt, hl, nb, kmax), dtype=torch.int32, device=dev)
    _check_tensor(cnt, "visit_cnt", shape=(bt, hl, nb), dtype=torch.int32, device=dev)
    _check_tensor(hrm, "hrm_cnt", shape=(bt, hl, nb), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", shape=q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty((bt, hq, n), dtype=torch.float32, device=q.device) if return_lse else None
    if pipeline is None:
        dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
        pipeline = _PIPELINES.get(dev)
        if pipeline is None:
            pipeline = _PIPELINES[dev] = Pipeline(dev)
    cur = torch.cuda.current_stream(q.device)
    pipeline.proxy.wait_stream(cur)
    pipeline.walk.wait_stream(cur)
    r = lib().cosa_prefill(ctypes.byref(shape), ctypes.byref(kparams), ctypes.byref(oparams),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                           ctypes.c_size_t(workspace.numel()), _ptr(idx), _ptr(cnt), _ptr(hrm),
                           ctypes.c_int(kmax), _ptr(out), _ptr(lse),
                           ctypes.c_int(head_chunks), _stream(pipeline.proxy), _stream(pipeline.walk),
                           ctypes.c_void_p(pipeline.event.cuda_event))
    cur.wait_stream(pipeline.walk)
    check(r)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_lists:
        res.append((idx, cnt, hrm))
    return res[0] if len(res) == 1 else tuple(res)


def dense(q, k, v, block: int = 128, causal: bool = True, scale: float = 0.0,
          return_lse: bool = False, out=None, seq_lens=None, stream=None):
    """Dense softmax attention (the baseline).  Returns out (and lse)."""
    torch = _torch()
    shape = make_shape(q, k, block, causal, scale, seq_lens)
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", shape=q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    r = lib().cosa_dense_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                              _stream(stream))
    check(r)
    return (out, lse) if return_lse else out
