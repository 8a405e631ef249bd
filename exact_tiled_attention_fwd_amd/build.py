"""Build the HIP library ``libfa.so`` for gfx950 in-tree with hipcc.

Run ``python -m exact_tiled_attention_fwd_amd.build`` (or call ``build()``).
Every call recompiles. Objects go to ``_build/`` next to this file; the
shared library lands beside this file so the binding finds it.

``build(sanitize=True)`` builds ``libfa_hostsan.so``: the same library with
its host code (argument validation, planning, dispatch) compiled under
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is
unchanged. It is loaded only by the host-sanitizer test, with the sanitizer
runtime preloaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libfa.so")
HOSTSAN_LIB_PATH = os.path.join(HERE, "libfa_hostsan.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fwd_fp8.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: the compiler may not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument",
]

# Sanitizers for the host pass only (each flag right after -Xarch_host).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag: that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, sanitize: bool = False) -> str:
    bdir = os.path.join(BUILD_DIR, "hostsan") if sanitize else BUILD_DIR
    out = HOSTSAN_LIB_PATH if sanitize else LIB_PATH
    extra = HOST_SANITIZE if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = out + ".tmp"
    link_extra = ["-shared-libsan", *HOST_SANITIZE[:2]] if sanitize else []
    outs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]))
    os.replace(tmp, out)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
