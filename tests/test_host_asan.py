"""The library's host code under AddressSanitizer (CPU only, no device call)."""
import os
import subprocess


def test_c_caller_host_checks_under_address_sanitizer(tmp_path):
    """The host code of the library (validation, sizing, workspace layout) and the C caller's
    host-only path built with AddressSanitizer: no invalid access and no leak is reported."""
    from block_sparse_attention_kap_amd.build import build_host_asan
    exe = build_host_asan(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23")
    r = subprocess.run([exe, "--host-only"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=120, env=env)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, out
    assert "c abi host checks ok" in out
    assert "AddressSanitizer" not in out
