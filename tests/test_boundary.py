"""C-ABI boundary tests that need no GPU.

The library must load, export every function include/cosa.h declares, keep the
struct layouts the binding assumes, and reject invalid arguments on the host
before any HIP call.  Calls here return from argument validation, so no kernel
is launched and no device memory is touched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_kap_amd as cosa
from block_sparse_attention_kap_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cosa.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cosa.lib_path()):
        from block_sparse_attention_kap_amd.build import build
        build()
    return cosa.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cosa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", cosa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (cosa_[a-z_]+)\b", out))
    assert set(declared) <= exported
    for name in declared:
        assert getattr(L, name) is not None


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %d\\n", sizeof(cosa_shape), offsetof(cosa_shape, scale), offsetof(cosa_shape, dtype), offsetof(cosa_shape, causal), offsetof(cosa_shape, seq_lens), COSA_MAX_VARLEN_BATCH);
  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(cosa_kap_params), offsetof(cosa_kap_params, mass), offsetof(cosa_kap_params, force_diag), offsetof(cosa_kap_params, sel_mode), offsetof(cosa_kap_params, order_mode), offsetof(cosa_kap_params, share_kv));
  printf("%zu %zu %zu %zu %zu\\n", sizeof(cosa_osk_params), offsetof(cosa_osk_params, skip_mode), offsetof(cosa_osk_params, skip_param), offsetof(cosa_osk_params, vote_rows), offsetof(cosa_osk_params, shared_lists));
  return 0;
}}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    S, K, P = _lib.Shape, _lib.KapParams, _lib.OskParams
    want = [ctypes.sizeof(S), S.scale.offset, S.dtype.offset, S.causal.offset, S.seq_lens.offset,
            _lib.COSA_MAX_VARLEN_BATCH,
            ctypes.sizeof(K), K.mass.offset, K.force_diag.offset, K.sel_mode.offset, K.order_mode.offset,
            K.share_kv.offset,
            ctypes.sizeof(P), P.skip_mode.offset, P.skip_param.offset, P.vote_rows.offset,
            P.shared_lists.offset]
    assert [int(x) for x in got] == want


def test_status_strings(L):
    for s in (0, -1, -2, -3, -99):
        assert isinstance(L.cosa_status_string(s), bytes)
    assert L.cosa_status_string(0) == b"ok"
    assert L.cosa_version() >= 10000


def _shape(**kw):
    d = dict(batch=1, q_heads=32, kv_heads=8, seq_len=131072, head_dim=128, block=128, causal=1,
             scale=0.0, dtype=_lib.COSA_BF16)
    d.update(kw)
    return _lib.Shape(**d)


def test_grid_row_limit(L):
    # the proxy launches one grid row per (batch entry, query head): at most 65535 of them
    ok = _shape(batch=2047, q_heads=32, kv_heads=8, seq_len=1024)
    assert L.cosa_list_capacity(ctypes.byref(ok), ctypes.c_double(0.5)) == 4
    big = _shape(batch=2048, q_heads=32, kv_heads=8, seq_len=1024)
    assert L.cosa_list_capacity(ctypes.byref(big), ctypes.c_double(0.5)) == -2
    assert L.cosa_dense_attn(ctypes.byref(big), 256, 256, 256, 256, None, None) == -2


def test_ragged_lengths_accepted(L):
    # block need not divide seq_len: the last block is partial (ceil(N / B) blocks)
    assert L.cosa_list_capacity(ctypes.byref(_shape(seq_len=1000)), ctypes.c_double(1.0)) == 8
    assert L.cosa_list_capacity(ctypes.byref(_shape(seq_len=100)), ctypes.c_double(0.5)) == 1
    assert L.cosa_list_capacity(ctypes.byref(_shape(seq_len=4096 * 128 + 1)), ctypes.c_double(0.5)) == -2
    sh = _shape(seq_len=1000)
    n = L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap()))
    np_ = -(-1000 // 32)                      # pooled rows per head, last group partial
    a256 = lambda x: (x + 255) // 256 * 256
    assert n == a256(32 * np_ * 128 * 2) + a256(8 * np_ * 128 * 2) + a256(32 * np_ * 8 * 4)
    # pages are whole blocks: paging a ragged sequence is unsupported
    r = L.cosa_ordered_sparse_attn(ctypes.byref(sh), ctypes.byref(_osk()), 256, 256, 256, 256, 256,
                                   4, 256, 256, None, None, None, None)
    assert r == -2


def _varlen(lens, **kw):
    sh = _shape(batch=len(lens), **kw)
    arr = (ctypes.c_int32 * len(lens))(*lens)
    sh._lens = arr
    sh.seq_lens = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return sh


def test_varlen_validation(L):
    ok = _varlen([8192, 1000, 128], seq_len=8192)
    assert L.cosa_list_capacity(ctypes.byref(ok), ctypes.c_double(0.5)) == 32
    for lens, code in (([8192, 0, 128], -1), ([8193, 100], -1), ([-5], -1),
                       ([100] * 129, -2)):
        sh = _varlen(lens, seq_len=8192)
        assert L.cosa_list_capacity(ctypes.byref(sh), ctypes.c_double(0.5)) == code, lens
        assert L.cosa_dense_attn(ctypes.byref(sh), 16, 16, 16, 16, None, None) == code, lens
    # a page table needs whole blocks in every entry
    r = L.cosa_ordered_sparse_attn(ctypes.byref(ok), ctypes.byref(_osk()), 256, 256, 256, 256, 256,
                                   4, 256, 256, None, None, None, None)
    assert r == -2


def test_list_capacity(L):
    assert L.cosa_list_capacity(ctypes.byref(_shape()), ctypes.c_double(0.1)) == 103
    assert L.cosa_list_capacity(ctypes.byref(_shape(seq_len=8192)), ctypes.c_double(0.3)) == 20
    assert L.cosa_list_capacity(ctypes.byref(_shape(seq_len=32768)), ctypes.c_double(0.2)) == 52
    assert L.cosa_list_capacity(ctypes.byref(_shape(q_heads=28, kv_heads=4, block=64)),
                                ctypes.c_double(0.08)) == 164
    assert L.cosa_list_capacity(ctypes.byref(_shape()), ctypes.c_double(1.5)) == -1
    assert L.cosa_list_capacity(ctypes.byref(_shape()), ctypes.c_double(0.0)) == -1
    assert L.cosa_list_capacity(None, ctypes.c_double(0.5)) == -1


@pytest.mark.parametrize("bad,code", [
    (dict(seq_len=0), -1), (dict(q_heads=30), -1), (dict(head_dim=96), -2),
    (dict(block=32), -2), (dict(dtype=7), -2), (dict(batch=0), -1), (dict(causal=2), -1),
    (dict(scale=-1.0), -1), (dict(scale=float("inf")), -1), (dict(seq_len=4097 * 128), -2),
])
def test_shape_validation(L, bad, code):
    sh = _shape(**bad)
    assert L.cosa_list_capacity(ctypes.byref(sh), ctypes.c_double(0.5)) == code
    assert L.cosa_dense_attn(ctypes.byref(sh), 16, 16, 16, 16, None, None) == code


def _kap(**kw):
    d = dict(budget=0.1, pool=0, pool_mode=0, agg_mode=0, sel_mode=0, mass=0.0, force_sink=0,
             force_diag=0, order_mode=0)
    d.update(kw)
    return _lib.KapParams(**d)


def test_workspace_bytes(L):
    sh = _shape()
    n = L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap()))
    np_ = 131072 // 32
    want = 32 * np_ * 128 * 2 + 8 * np_ * 128 * 2 + 32 * np_ * 1024 * 4
    assert n == want
    assert L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap(pool=3))) == 0
    assert L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap(budget=0.0))) == 0


def test_workspace_bytes_ragged_pitch(L):
    # 2216 tokens, block 128: 18 blocks, so each row of the proxy scores is padded to 20 floats
    # (16-byte aligned rows); pooled rows ceil(2216 / 32) = 70; each part 256-byte aligned
    sh = _shape(seq_len=2216)
    a256 = lambda x: (x + 255) // 256 * 256
    want = a256(32 * 70 * 128 * 2) + a256(8 * 70 * 128 * 2) + a256(32 * 70 * 20 * 4)
    assert L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap())) == want


@pytest.mark.parametrize("bad,code", [
    (dict(budget=0.0), -1), (dict(budget=1.01), -1), (dict(pool=3), -1), (dict(pool=256), -1),
    (dict(pool_mode=2), -1), (dict(agg_mode=5), -1), (dict(sel_mode=1, mass=0.0), -1),
    (dict(sel_mode=1, mass=1.5), -1), (dict(sel_mode=9), -1),
    (dict(force_sink=2), -1), (dict(order_mode=2), -1), (dict(share_kv=2), -1),
])
def test_proxy_param_validation(L, bad, code):
    sh = _shape(seq_len=8192)
    r = L.cosa_proxy_select(ctypes.byref(sh), ctypes.byref(_kap(**bad)), 256, 256, 256, 1 << 40,
                            256, 256, 256, None, 20, None)
    assert r == code


def test_shared_list_row_limit(L):
    # one list per KV head over 32 query heads x 64 pooled rows: above the 1024-row limit
    sh = _shape(seq_len=8192, kv_heads=1)
    r = L.cosa_proxy_select(ctypes.byref(sh), ctypes.byref(_kap(share_kv=1, pool=2)), 256, 256, 256,
                            1 << 40, 256, 256, 256, None, 20, None)
    assert r == -2
    assert L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(_kap(share_kv=1, pool=4))) > 0


def test_proxy_pointer_and_size_validation(L):
    sh = _shape(seq_len=8192)
    kp = _kap(budget=0.3)
    ws = L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(kp))
    call = lambda q=256, k=256, w=256, wb=ws, idx=256, cnt=256, hrm=256, kmax=20: \
        L.cosa_proxy_select(ctypes.byref(sh), ctypes.byref(kp), q, k, w, wb, idx, cnt, hrm, None,
                            kmax, None)
    assert call(q=None) == -1
    assert call(k=None) == -1
    assert call(w=None) == -1
    assert call(idx=None) == -1
    assert call(cnt=None) == -1
    assert call(hrm=None) == -1
    assert call(w=512 + 16) == -1              # workspace not 256-byte aligned
    assert call(q=256 + 2) == -1               # q not 16-byte aligned
    assert call(wb=ws - 1) == -1               # workspace too small
    assert call(kmax=19) == -1                 # below the list capacity
    assert call(kmax=65) == -1                 # above nb


def _osk(**kw):
    d = dict(tight_budget=0.05, cap_mode=0, skip_mode=2, skip_param=1e-3, vote_rows=0)
    d.update(kw)
    return _lib.OskParams(**d)


@pytest.mark.parametrize("bad", [
    dict(tight_budget=0.0), dict(tight_budget=2.0), dict(cap_mode=2), dict(skip_mode=3),
    dict(skip_mode=2, skip_param=0.0), dict(skip_mode=2, skip_param=-1.0),
    dict(skip_mode=1, skip_param=float("nan")), dict(vote_rows=16), dict(vote_rows=64),
    dict(shared_lists=2),
])
def test_osk_param_validation(L, bad):
    sh = _shape(seq_len=8192)
    r = L.cosa_ordered_sparse_attn(ctypes.byref(sh), ctypes.byref(_osk(**bad)), 256, 256, 256, 256,
                                   256, 20, None, 256, None, None, None, None)
    assert r == -1


def test_osk_pointer_validation(L):
    sh = _shape(seq_len=8192)
    op = _osk()
    call = lambda q=256, k=256, v=256, idx=256, cnt=256, kmax=20, out=256: \
        L.cosa_ordered_sparse_attn(ctypes.byref(sh), ctypes.byref(op), q, k, v, idx, cnt, kmax,
                                   None, out, None, None, None, None)
    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(idx=None), dict(cnt=None),
               dict(out=None), dict(kmax=0), dict(kmax=65), dict(out=264)):
        assert call(**kw) == -1, kw
    assert L.cosa_ordered_sparse_attn(ctypes.byref(sh), None, 256, 256, 256, 256, 256, 20, None,
                                      256, None, None, None, None) == -1


def test_prefill_validation(L):
    # every rejected call returns before its first HIP call (no GPU needed)
    sh = _shape(seq_len=8192)
    kp = _kap(budget=0.3)
    ws = L.cosa_kap_workspace_bytes(ctypes.byref(sh), ctypes.byref(kp))

    def call(kap=kp, osk=None, q=256, k=256, v=256, w=256, wb=ws, idx=256, cnt=256, hrm=256,
             kmax=20, out=256, chunks=4, event=256):
        o = _osk(tight_budget=0.15) if osk is None else osk
        return L.cosa_prefill(ctypes.byref(sh), ctypes.byref(kap), ctypes.byref(o), q, k, v, w, wb,
                              idx, cnt, hrm, kmax, out, None, chunks, None, None, event)

    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(w=None), dict(idx=None),
               dict(cnt=None), dict(hrm=None), dict(out=None), dict(event=None),
               dict(w=512 + 16), dict(q=256 + 2), dict(wb=ws - 1), dict(kmax=19), dict(kmax=65),
               dict(chunks=0), dict(chunks=3), dict(chunks=16),           # 8 KV heads
               dict(osk=_osk(shared_lists=1)),                            # lists per query head
               dict(kap=_kap(budget=0.3, share_kv=1)),                    # lists per KV head
               dict(osk=_osk(tight_budget=0.0)), dict(kap=_kap(budget=0.0))):
        assert call(**kw) == -1, kw


def test_binding_has_no_cpu_fallback(monkeypatch, tmp_path):
    monkeypatch.setenv("COSA_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(ImportError):
        _lib.lib()


def _c_caller():
    """The plain C caller (tests/c_abi), built with the library; built here if missing."""
    from block_sparse_attention_kap_amd import build as _build
    if not os.path.exists(_build.C_CHECK_BIN):
        _build.build_c_check()
    return _build.C_CHECK_BIN


def test_c_caller_host_checks():
    """The ABI from C without Python: sizing helpers, status strings and argument
    validation (every invalid call returns its status before any device work)."""
    r = subprocess.run([_c_caller(), "--host-only"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=60)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, out
    assert "c abi host checks ok" in out


@pytest.mark.gpu
def test_c_caller_device():
    """The ABI from C on the GPU: proxy, ordered walk and dense on a ragged GQA problem; at
    full budgets with the skip test off the lists are permutations of the candidates and
    the walk equals the dense attention."""
    print("c caller: proxy + ordered walk + dense from C", flush=True)
    r = subprocess.run([_c_caller()], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=120)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, out
    assert "c abi device checks ok" in out, out


@pytest.mark.parametrize("bad,code", [
    (dict(budget=0.0), -1), (dict(pool=3), -1), (dict(share_kv=2), -1), (dict(sel_mode=9), -1),
])
def test_noalloc_param_validation(L, bad, code):
    # the entry point that allocates nothing validates like cosa_proxy_select, before any HIP call
    sh = _shape(seq_len=8192)
    r = L.cosa_proxy_select_noalloc(ctypes.byref(sh), ctypes.byref(_kap(**bad)), 256, 256, 256, 256,
                                    256, None, 20, None)
    assert r == code


def test_noalloc_rejects_problems_larger_than_its_scratch(L):
    """The static scratch holds COSA_NOALLOC_SCRATCH_MIB MiB.  A query head whose block scores
    alone exceed it (4096 blocks of 128: 16384 pooled rows x 4096 blocks x 4 bytes = 256 MiB),
    or a shared list whose KV head with all its query heads exceeds it, is refused with
    COSA_ERR_SCRATCH before any HIP call; arguments that are invalid anyway stay INVALID_ARG."""
    assert _lib.COSA_NOALLOC_SCRATCH_MIB == 128
    big = _shape(q_heads=1, kv_heads=1, seq_len=4096 * 128)
    r = L.cosa_proxy_select_noalloc(ctypes.byref(big), ctypes.byref(_kap()), 256, 256, 256, 256,
                                    256, None, 410, None)
    assert r == _lib.COSA_ERR_SCRATCH
    assert L.cosa_status_string(r).startswith(b"problem too large")
    # 128K, 32/8 heads, shared lists: the layer's workspace exceeds the array, but one KV head's
    # slice (4 query heads x 4096 pooled rows x 1024 blocks x 4 bytes = 64 MiB, plus pooled
    # rows) fits; at 256K one KV head's slice needs 4 x 8192 x 2048 x 4 bytes = 256 MiB
    ok = _shape(seq_len=131072)
    assert L.cosa_kap_workspace_bytes(ctypes.byref(ok), ctypes.byref(_kap(share_kv=1))) > 128 << 20
    sh = _shape(seq_len=262144)
    r = L.cosa_proxy_select_noalloc(ctypes.byref(sh), ctypes.byref(_kap(share_kv=1)), 256, 256,
                                    256, 256, 256, None, 205, None)
    assert r == _lib.COSA_ERR_SCRATCH
    # null output pointer: an invalid argument whatever the size
    r = L.cosa_proxy_select_noalloc(ctypes.byref(big), ctypes.byref(_kap()), 256, 256, None, 256,
                                    256, None, 410, None)
    assert r == -1

