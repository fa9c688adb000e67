"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/oracle.cpp) built with -fsanitize=address,undefined, every
  finding fatal, runs the oracle pin tests in a child process with GCC's libasan
  preloaded (PKV_ORACLE_LIBRARY selects that build).
* The library's host side (libpkv_hostsan.so, made by build(): the API unit's host
  code, where every entry point checks its arguments and sets up its launches,
  compiled with the same sanitizers) runs the C-ABI tests in a child process with
  clang's AddressSanitizer runtime preloaded (PKV_LIBRARY selects that build).

A finding ends the child with an error and a report; either fails the test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(tests, preload, extra_env):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    cmd = [sys.executable, "-m", "pytest", *[os.path.join(ROOT, "tests", t) for t in tests],
           "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=900)
    out = res.stdout
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    import oracle

    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()
    out = _child(["test_oracle_pins.py"], asan, {"PKV_ORACLE_LIBRARY": lib})
    assert " passed" in out


def test_the_sanitized_oracle_reports_a_planted_overflow(tmp_path):
    """The harness is live: a copy of the oracle whose fp8 decoding loop runs one
    element past its buffers must end the sanitized child with a report."""
    import oracle

    src = open(os.path.join(ROOT, "oracle", "oracle.cpp")).read()
    good = "for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_float(codes[i]);"
    assert src.count(good) == 1
    bad_src = tmp_path / "oracle_bad.cpp"
    bad_src.write_text(src.replace(good, good.replace("i < n", "i <= n")))
    lib = str(tmp_path / "liboracle_bad.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer", str(bad_src),
                    "-o", lib], check=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()
    # arrays large enough to come straight from malloc (the sanitizer's redzones)
    code = ("import numpy as np, oracle; "
            "oracle.fp8_e4m3_to_f32(np.arange(1 << 16, dtype=np.int64).astype(np.uint8))")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=300,
                         env=dict(os.environ, LD_PRELOAD=asan, PKV_ORACLE_LIBRARY=lib,
                                  **SAN_ENV))
    assert res.returncode != 0 and "AddressSanitizer" in res.stdout, res.stdout[-2000:]


def test_c_abi_host_checks_pass_under_asan_and_ubsan():
    from paged_kv_cache_280_amd import build

    if not os.path.exists(build.HOSTSAN_LIB):
        pytest.fail("libpkv_hostsan.so is not built; run python -m paged_kv_cache_280_amd.build")
    out = _child(["test_abi_cpu.py"], build.sanitizer_runtime(),
                 {"PKV_LIBRARY": build.HOSTSAN_LIB})
    assert " passed" in out
