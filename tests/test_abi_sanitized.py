"""The C-ABI checks of test_abi.py again, against the library built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code (argument
validation, workspace-size queries and every error path of the C entry points
run instrumented; a sanitizer report ends the run with a failure).

The sanitized build links the shared sanitizer runtime, so the checks run in a
child interpreter that preloads it and loads that build through DFLASH_LIB.
No GPU is involved: on a GPU-less host every fully valid call stops at the
device check."""

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_library():
    from block_draft_verification_amd import _build  # imported here: build tooling only
    srcs = glob.glob(os.path.join(_build.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    lib = _build.SAN_OUT
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(f) for f in srcs):
        _build.build(sanitize=True)
    return lib, _build.san_runtime()


def test_abi_checks_under_host_sanitizers():
    lib, rt = _sanitized_library()
    assert os.path.exists(rt), rt
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report_load" in undef and "__ubsan_handle" in undef, "library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, DFLASH_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child really loads the sanitized build
    probe = ("import block_draft_verification_amd as d; d.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libdflash_san.so' in m and 'libdflash.so' not in m.replace('libdflash_san.so', '')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out and "skipped" not in out, out[-3000:]
