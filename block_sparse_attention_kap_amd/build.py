"""Compile libcosa.so (HIP kernels + C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcosa.so")
SOURCES = ["api.cpp", "kap_pool.hip", "kap_score.hip", "kap_select.hip", "attn.hip"]
ARCH = "gfx950"
# per-source extras: the score kernel keeps its MFMA accumulator in ordinary VGPRs (left to
# itself the compiler picks AGPRs there and copies every tile out of them, twice)
EXTRA = {"kap_score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # no packed fp32 arithmetic (v_pk_*_f32) in the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libcosa.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmd = [cc] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc] + flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(x for x in out.splitlines() if "packed-fp32-ops" not in x)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{o}" for s, o in failed))
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    build_c_check()
    return LIB


def build_host_asan(outdir: str) -> str:
    """A copy of the library and of the plain C caller whose host code (argument validation,
    workspace layout, launch set-up) is built with AddressSanitizer, for a CPU test of the
    host-only path.  Device code is built as usual (the sanitizer is for the host only).
    Returns the path of the sanitized C caller."""
    os.makedirs(outdir, exist_ok=True)
    cc = hipcc()
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(outdir, src.replace(".", "_") + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else EXTRA.get(src, [])
        cmd = [cc] + flags() + asan + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed on {src}:\n{out}")
    lib = os.path.join(outdir, "libcosa.so")
    r = subprocess.run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-fsanitize=address",
                        "-o", lib] + objs, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("asan link failed:\n" + r.stdout.decode(errors="replace"))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(outdir, "cosa_c_abi_check")
    cmd = [os.path.join(rocm, "llvm", "bin", "clang"), "-std=c11", "-O1", "-g", "-fsanitize=address",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), C_CHECK_SRC, "-o", exe, "-L", outdir, "-lcosa",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + outdir,
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("asan C caller build failed:\n" + r.stdout.decode(errors="replace"))
    return exe


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "cosa_c_abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "cosa_c_abi_check")


def build_c_check() -> str:
    """The plain C caller of the library (tests/c_abi): gcc against the HIP runtime's C API,
    linked to this libcosa.so by relative rpath."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_CHECK_SRC, "-o", C_CHECK_BIN + ".tmp",
           "-L", PKG, "-lcosa", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../block_sparse_attention_kap_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("C check build failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(C_CHECK_BIN + ".tmp", C_CHECK_BIN)
    return C_CHECK_BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
