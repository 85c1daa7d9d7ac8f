"""Compile the HIP sources of the library into ``libdflash.so`` (gfx950).

Each translation unit is compiled to an object with hipcc, then linked into
one shared library next to this file.  Used by ``__graft_entry__.build()`` and
runnable as ``python -m block_draft_verification_amd._build``.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdflash.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "conv2tap.hip", "conv_proj.hip", "head_topk.hip", "select_path.hip", "verify.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


# The host-sanitized variant (AddressSanitizer + UndefinedBehaviorSanitizer on
# the host code only; the device code is built as usual).  It links the shared
# sanitizer runtime, which a process must preload (SAN_RUNTIME) to load it.
SAN_OUT = os.path.join(HERE, "libdflash_san.so")
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-shared-libsan", "-O1",
]


def san_runtime():
    """Path of the shared AddressSanitizer runtime of hipcc's host compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    return r.stdout.strip()


def build(verbose=False, sanitize=False):
    out, bdir = (SAN_OUT, SAN_BUILD) if sanitize else (OUT, BUILD)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".", "_") + ".o")
        cmd = [HIPCC] + FLAGS + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + extra + ["-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
