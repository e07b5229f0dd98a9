"""Build step for libmha.so (the gfx950 HIP library behind include/mha.h).

    python -m head_attention_forward_flash_amd.build [--save-temps DIR]

Compiles every csrc/*.hip translation unit with hipcc for gfx950 and links
them into head_attention_forward_flash_amd/libmha.so (in-tree, next to this
file).  Cross-compiles on a machine without a GPU.
"""

from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_PATH = os.path.join(PKG_DIR, "libmha.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU forms are kept out of the generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def check_exports(path: str) -> None:
    """Refuse a library whose host objects reference kernel stubs they never defined.

    A host-side compile that silently drops a kernel's launch stub leaves an undefined
    symbol that only shows up when the library is loaded; catch it at build time.
    """
    nm = shutil.which("nm")
    if nm is None:
        return
    r = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "_ZN3mha" in ln]
    if missing:
        raise RuntimeError("libmha.so has undefined internal symbols: " + ", ".join(missing))


def build(verbose: bool = False, save_temps: str | None = None, jobs: int = 8) -> str:
    cc = hipcc()
    srcs = sources()
    tmp = tempfile.mkdtemp(prefix="mha_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            if save_temps:
                os.makedirs(save_temps, exist_ok=True)
                cmd += ["-save-temps"]
                cwd = save_temps
            else:
                cwd = tmp
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")
            warn = (r.stderr or "").strip()
            if verbose and warn:
                print(warn, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            objs = list(ex.map(compile_one, srcs))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        check_exports(out_tmp)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="directory for .s/.bc intermediates")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=8)
    a = ap.parse_args()
    path = build(verbose=a.verbose, save_temps=a.save_temps, jobs=a.jobs)
    print(path)


if __name__ == "__main__":
    main()
