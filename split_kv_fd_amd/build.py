"""Build libfd.so (the HIP library behind include/fd.h) in-tree for gfx950.

    python -m split_kv_fd_amd.build        # or: python split_kv_fd_amd/build.py

Every source is compiled by hipcc for gfx950 only; packed-fp32 VALU forms are
switched off for device code (the compiler otherwise forms them from plain
float code).  Objects go to split_kv_fd_amd/_build/, the library to
split_kv_fd_amd/libfd.so.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfd.so")
SOURCES = ["fd_api.cpp", "fd_split_valu.hip", "fd_split_mfma.hip", "fd_combine.hip", "fd_prefill.hip",
           "fd_noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def build(verbose: bool = False, out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile every source and link `out`.  `defines` are extra -D flags
    (compile-time variants); objects go to `build_dir`."""
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *CFLAGS, *[f"-D{d}" for d in defines], *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        # The host pass does not know the device-only feature flag; that note is noise.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
