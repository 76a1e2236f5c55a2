"""Build libdcp.so (HIP kernels + C ABI) in-tree with hipcc for gfx950."""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdcp.so")
# host-sanitized variant for the CPU ABI tests (never loaded on a GPU run)
LIB_SANITIZED = os.path.join(BUILD, "libdcp_asan.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host half of dcp_api.cpp only: every
# -fsanitize goes to the host pass (-Xarch_host), so no device code is instrumented
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer", "-g"]

# (source, object name, extra hipcc flags)
SOURCES = [
    ("dcp_api.cpp", "dcp_api", []),
    ("k_util.hip", "k_util", []),
    ("k_gqa_valu.hip", "k_gqa_valu", []),
    ("k_gqa_mfma.hip", "k_gqa_mfma", []),
    ("k_gqa_chunk.hip", "k_gqa_chunk", []),
    ("k_mla_mfma.hip", "k_mla_mfma", []),
    ("k_mla_ring.hip", "k_mla_ring", []),
    ("k_mla_pair16.hip", "k_mla_pair16", []),
]

# -packed-fp32-ops keeps hipcc from emitting packed fp32 VALU ops (v_pk_*_f32).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
               "-Wno-unused-function", "-Wno-pass-failed", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libdcp.so")
    return path


def _compile(spec, verbose: bool, suffix: str = "") -> str:
    src, name, extra = spec
    obj = os.path.join(BUILD, name + suffix + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "warning generated" not in l
                    and "warnings generated" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out:
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdcp.so next to this file; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a sanitized library needs preloaded."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so was not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """libdcp_asan.so under _build/: dcp_api.cpp (the host-side validation, planning and
    workspace layout) built with ASan + UBSan on the host pass, linked with the kernels as
    they are. For CPU tests only; load it with the ASan runtime preloaded."""
    os.makedirs(BUILD, exist_ok=True)
    specs = [(src, name, extra + (SANITIZE_FLAGS if src == "dcp_api.cpp" else []))
             for src, name, extra in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(specs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, "_asan"), specs))
    tmp = LIB_SANITIZED + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
                          "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                          "-fsanitize=undefined", "-shared-libasan", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_SANITIZED)
    return LIB_SANITIZED


if __name__ == "__main__":
    print(build(verbose=True))
