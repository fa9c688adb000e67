"""Build the HIP library ``libpkv.so`` in place (gfx950 only).

Run as ``python -m paged_kv_cache_280_amd.build`` or call ``build()``.  The
library is rebuilt on every call: each source compiles to an object file in
parallel (the decode kernel instances are spread over several sources), then one
link step makes the shared library.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpkv.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"
# hipcc's host pass does not know the packed-fp32 feature and says so
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def compile_command(src: str, obj: str):
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-c",
            # packed fp32 VALU ops stay off: plain float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), src, "-o", obj]


def link_command(objs, out: str):
    return [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msg = "\n".join(l for l in res.stdout.splitlines() if _NOISE not in l)
    return res.returncode, msg


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = "%d" % os.getpid()
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + "." + tag + ".o")
        jobs.append((compile_command(src, obj), obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), flush=True)
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: _run(j[0]), jobs))
    objs = [obj for _, obj in jobs]
    try:
        for (cmd, _), (rc, msg) in zip(jobs, results):
            if rc != 0:
                raise RuntimeError("hipcc failed (%d): %s\n%s" % (rc, cmd[-3], msg))
            if msg.strip() and verbose:
                print(msg)
        tmp = LIB + ".tmp" + tag
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msg = _run(cmd)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, msg))
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
