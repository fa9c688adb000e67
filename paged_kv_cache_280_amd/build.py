"""Build the HIP library ``libpkv.so`` in place (gfx950 only).

Run as ``python -m paged_kv_cache_280_amd.build`` or call ``build()``.  The
library is rebuilt on every call: each source compiles to an object file in
parallel (the decode kernel instances are spread over several sources), then one
link step makes the shared library.

``build(timeline=True)`` (``--timeline``) makes the measurement variant
``libpkv_timeline.so``: the same sources with PKV_TIMELINE defined, whose decode
kernel also stamps each worker's entry, plan, first tile and end times into the
workspace (read by ``bench.py --timeline``).  ``build_stream_probe()`` makes
``libpkv_stream.so``, the HBM read-stream probe that bench.py reports as the
attainable bandwidth.

Every ``build()`` also links ``libpkv_hostsan.so``: the same kernel objects with the API
translation unit (``pkv_api.hip``: every entry point's argument checks and launch set-up)
compiled again with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
only.  The CPU tests load it (``PKV_LIBRARY``) under the sanitizer runtime to run the
host-side checks; it is never the product library.
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
TIMELINE_LIB = os.path.join(PKG, "libpkv_timeline.so")
STREAM_LIB = os.path.join(PKG, "libpkv_stream.so")
STREAM_SRC = os.path.join(PKG, "probe", "pkv_stream.hip")
HOSTSAN_LIB = os.path.join(PKG, "libpkv_hostsan.so")
API_SRC = os.path.join(PKG, "csrc", "pkv_api.hip")
# host-side sanitizers only (each flag behind -Xarch_host: the device code is unchanged)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
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


def compile_command(src: str, obj: str, defines=()):
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-c",
            # packed fp32 VALU ops stay off: plain float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # atomics stay as written: the wave-level rewrite of single-lane atomics
            # reads their result back at once, which would drain the decode kernel's
            # tile loads at every chunk claim
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-Wall", "-Wno-unused-result", *["-D" + x for x in defines],
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), src, "-o", obj]


def link_command(objs, out: str):
    return [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msg = "\n".join(l for l in res.stdout.splitlines() if _NOISE not in l)
    return res.returncode, msg


def build(verbose: bool = False, timeline: bool = False) -> str:
    if timeline:
        return _build_lib(sources(), TIMELINE_LIB, ("PKV_TIMELINE=1",), verbose)
    return _build_lib(sources(), LIB, (), verbose, hostsan=HOSTSAN_LIB)


def build_stream_probe(verbose: bool = False) -> str:
    return _build_lib([STREAM_SRC], STREAM_LIB, (), verbose)


def _build_lib(srcs, lib: str, defines, verbose: bool, hostsan=None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = "%d.%s" % (os.getpid(), os.path.basename(lib)[:-3])
    jobs = []
    for src in srcs:
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + "." + tag + ".o")
        jobs.append((compile_command(src, obj, defines), obj))
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
        tmp = lib + ".tmp" + tag
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msg = _run(cmd)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, msg))
        os.replace(tmp, lib)
        if hostsan:
            _link_hostsan(jobs, hostsan, tag, defines, verbose)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return lib


def _link_hostsan(jobs, out: str, tag: str, defines, verbose: bool) -> None:
    """``out``: the objects of ``jobs`` with the API unit recompiled under the host
    sanitizers (its object joins the others; removed with them)."""
    obj = os.path.join(OBJ_DIR, "pkv_api.%s.hostsan.o" % tag)
    cmd = compile_command(API_SRC, obj, defines)
    cmd = cmd[:-3] + HOST_SANITIZE + cmd[-3:]   # before "<src> -o <obj>"
    try:
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msg = _run(cmd)
        if rc != 0:
            raise RuntimeError("hipcc failed (%d): %s\n%s" % (rc, API_SRC, msg))
        objs = [o for c, o in jobs if c[-3] != API_SRC] + [obj]
        tmp = out + ".tmp" + tag
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-shared-libsan",
               *HOST_SANITIZE[:4], *objs, "-o", tmp]
        rc, msg = _run(cmd)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, msg))
        os.replace(tmp, out)
    finally:
        if os.path.exists(obj):
            os.remove(obj)


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the host-sanitized library needs
    (preloaded into the process that loads it)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found under " + rocm)
    return found[-1]


if __name__ == "__main__":
    if "--timeline" in sys.argv:
        print(build(verbose="-v" in sys.argv, timeline=True))
    elif "--stream-probe" in sys.argv:
        print(build_stream_probe(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
