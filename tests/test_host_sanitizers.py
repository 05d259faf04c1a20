"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The host side of libmoe_mlp.so (argument validation, workspace planning,
launch selection) is built a second time with host-only ASan + UBSan
instrumentation (the gfx950 device code is compiled as usual and not
instrumented), and the C-ABI checks of test_abi.py run against that build in a
child process that preloads the sanitizer runtime.  Any invalid memory access
or undefined behaviour on those paths (every validation error path, the
workspace-size and stage-name queries) aborts the child.

The instrumented build goes to _build/asan/ and is reused while the sources
hash to the value stamped beside it.
"""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libmoe_mlp.so")
STAMP = os.path.join(OUT, "sources.sha256")


def _sources():
    csrc = os.path.join(ROOT, "routed_expert_mlp_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    return files + [os.path.join(ROOT, "include", "moe_mlp.h")]


def _digest():
    h = hashlib.sha256()
    for p in _sources():
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def _asan_runtime(hipcc):
    """The shared ASan runtime of hipcc's clang (it carries the UBSan handlers too)."""
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
        return p
    base = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "lib", "clang")
    if os.path.isdir(base):
        for v in sorted(os.listdir(base), reverse=True):
            p = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(p):
                return p
    return None


def _build(hipcc):
    digest = _digest()
    if os.path.exists(LIB) and os.path.exists(STAMP) and open(STAMP).read().strip() == digest:
        return
    from routed_expert_mlp_amd import build as B
    os.makedirs(OUT, exist_ok=True)
    # sanitizer flags for the host pass only (each -fsanitize= behind -Xarch_host)
    host = ["-O1", "-g", "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-shared-libsan", "-fno-omit-frame-pointer"]
    flags = [f for f in B.HIPCC_FLAGS if f != "-Wall"]
    cmd = [hipcc] + flags + [x for f in host for x in ("-Xarch_host", f)] + \
          ["-I", os.path.join(ROOT, "include"), B.SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    os.replace(LIB + ".tmp", LIB)
    with open(STAMP, "w") as f:
        f.write(digest + "\n")


DRIVER = r"""
import sys
sys.path.insert(0, sys.argv[1])
from routed_expert_mlp_amd import capi
capi.LIB_PATH = sys.argv[2]
import pytest
sys.exit(pytest.main([sys.argv[3], "-q", "-x", "-p", "no:cacheprovider"]))
"""


@pytest.mark.slow
def test_abi_checks_under_host_asan_ubsan():
    from routed_expert_mlp_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _asan_runtime(hipcc)
    if rt is None:
        pytest.skip("no shared ASan runtime next to hipcc")
    _build(hipcc)
    # the build is instrumented: it calls the ASan and UBSan report handlers
    syms = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", DRIVER, ROOT, LIB, os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
