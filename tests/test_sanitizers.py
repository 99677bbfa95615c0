"""AddressSanitizer and UndefinedBehaviorSanitizer over the CPU code.

* The oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined
  (every report fatal) and its pin tests run against that build.
* The HIP library's host code -- the C ABI's argument checks, launch
  planning and dispatch -- is rebuilt with clang's sanitizers on the host
  pass only (-Xarch_host: device code is never instrumented), and the C-ABI
  tests, which exercise every check without a GPU, run against it.

Each run is a child pytest process with the sanitizer runtime preloaded
(Python itself is not instrumented) and leak detection off (the
interpreter's own allocations outlive it by design).  The builds go to a
temporary directory; the child swaps the library path before first use.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_OPTIONS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
               "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

ORACLE_TESTS = ["tests/test_oracle_region.py", "tests/test_oracle_rng.py",
                "tests/test_oracle_rs.py", "tests/test_oracle_variants.py",
                "tests/test_oracle_attention.py", "tests/test_oracle_accounting.py"]

# The child: point the package (or the oracle) at the sanitized build, then
# run pytest in-process.
CHILD = """
import sys
sys.path.insert(0, {root!r})
import {module} as m
m.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *{tests!r}]))
"""


def _run_child(module, lib, tests, preload):
    env = dict(os.environ, **SAN_OPTIONS, LD_PRELOAD=preload)
    code = CHILD.format(root=ROOT, module=module, lib=lib, tests=tests)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    from oracle import build as obuild
    lib = str(tmp_path / "libsp_oracle_san.so")
    obuild.build_oracle(lib, extra_flags=("-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                                          "-fno-sanitize-recover=all", "-g"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    out = _run_child("oracle", lib, ORACLE_TESTS, asan)
    assert " passed" in out


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_library_checks_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from dropout_region_amd import build as hbuild
    lib = str(tmp_path / "libsp_region_san.so")
    host = []
    for f in ("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-shared-libsan"):
        host += ["-Xarch_host", f]
    hbuild.build(out=lib, extra=host, build_dir=str(tmp_path / "objs"))
    out = _run_child("dropout_region_amd", lib, ["tests/test_abi.py"], rt)
    assert " passed" in out
