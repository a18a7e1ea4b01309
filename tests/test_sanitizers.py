"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds of the same sources: the C ABI library (uq_abi.cpp, whose host code does the
argument checks, the work planning and the workspace layout; the kernel objects are the
ordinary ones) with clang's sanitizers on its host side, and the fp64 oracle (uq_oracle.c)
with gcc's.  Each suite that exercises them -- the ABI checks of test_abi.py, and the
oracle's pins -- runs again in a child process with the matching ASan runtime preloaded;
any sanitizer report fails the test (UBSan is built not to recover, ASan aborts).
Leak checking is off: the Python interpreter keeps allocations until exit."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _exported(lib: str, symbol: str) -> bool:
    r = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True)
    return symbol in r.stdout


def _run_pytest(files, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", *files, "-q", "-m", "not gpu", "-p",
           "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_abi_checks_under_sanitizers(tmp_path):
    from quantized_paged_attention_amd import build
    lib = build.build_host_sanitized(str(tmp_path))
    assert _exported(lib, "__asan_report"), "the host code is not instrumented"
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    env = {"UQ_LIB": lib, "LD_PRELOAD": rt}
    # the child loads the sanitized build, not the in-tree one
    probe = ("from quantized_paged_attention_amd import uq; "
             "print(uq.load_library()._name)")
    e = dict(os.environ, **env, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=e, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == lib
    rc, out = _run_pytest(["tests/test_abi.py"], env)
    assert rc == 0 and not any(s in out for s in REPORTS), out[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    from oracle import oracle
    lib = oracle.build_sanitized(str(tmp_path))
    assert _exported(lib, "__asan_report"), "the oracle is not instrumented"
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True, check=True).stdout.strip()
    if not os.path.isabs(rt):
        pytest.skip("gcc's libasan is not installed")
    files = ["tests/test_oracle_codecs.py", "tests/test_oracle_attention.py",
             "tests/test_oracle_index.py", "tests/test_oracle_mtp.py",
             "tests/test_oracle_pertoken.py"]
    rc, out = _run_pytest(files, {"UQ_ORACLE_LIB": lib, "LD_PRELOAD": rt})
    assert rc == 0 and not any(s in out for s in REPORTS), out[-4000:]
