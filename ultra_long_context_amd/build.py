"""Build the HSA HIP library (libhsa.so) for gfx950 with hipcc, in-tree.

Each source compiles to its own object (in parallel; every kernel lives in
one translation unit, so no relocatable device code is needed), then hipcc
links the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhsa.so")
SOURCES = ["hsa_api.hip", "retrieve.hip", "attend.hip", "attend_chunk.hip", "attend_decode.hip",
           "landmarks.hip", "attend_global.hip", "backward.hip"]
ARCH = os.environ.get("HSA_OFFLOAD_ARCH", "gfx950")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
         "-Wno-unused-function",
         # packed fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_command(src: str, obj: str) -> list:
    return [hipcc()] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", out]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    tmpdir = tempfile.mkdtemp(prefix="hsa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_command(s, o) for s, o in zip(SOURCES, objs)]
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, out) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + out)
            if out.strip() and verbose:
                print(out)
        tmp = LIB + ".tmp%d" % os.getpid()
        rc, out = _run(link_command(objs, tmp))
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("hipcc link failed:\n" + out)
        os.replace(tmp, LIB)
        return LIB
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
