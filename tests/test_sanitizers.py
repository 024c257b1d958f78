"""Sanitizer runs of the host code (CPU only).

* The oracle (sa_oracle.c) and the input generator (synth.c) are rebuilt with
  gcc's AddressSanitizer and UndefinedBehaviorSanitizer (every error fatal) and
  the oracle and generator pin tests run again on those builds, in a child
  process with the ASan runtime preloaded.
* libsa.so is rebuilt with its host code instrumented the same way (clang,
  -Xarch_host before every sanitizer flag: no GPU code is instrumented) and the
  C-ABI tests, which drive the host-side argument validation, sizing and
  planning of every entry point without a GPU, run again on it.
A child that reports a sanitizer error exits nonzero (halt on error), and its
output is searched for reports as well.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _child(env_extra, tests):
    env = dict(os.environ, PYTHONPATH=ROOT, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    lo = oracle.build(out=str(tmp_path / "liboracle_asan.so"), sanitize=True)
    ls = synth.build(out=str(tmp_path / "libsynth_asan.so"), sanitize=True)
    out = _child({"LD_PRELOAD": libasan, "SA_ORACLE_LIB": lo, "SA_SYNTH_LIB": ls},
                 sorted(os.path.basename(p) for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
                 + ["test_synth.py"])
    print(out.strip().splitlines()[-1])


def test_library_host_code_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime")
    from query_aware_sparse_min_amd import build as sa_build
    lib = sa_build.build(out=str(tmp_path / "libsa_host_asan.so"), sanitize_host=True)
    out = _child({"LD_PRELOAD": rt[-1], "SA_LIB_PATH": lib}, ["test_abi.py"])
    print(out.strip().splitlines()[-1])
