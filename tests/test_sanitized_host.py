"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument validation, workspace sizing, the no-allocation entry
point's capacity check) and blockmask.cpp (the block-mask builder and its
transpose) are rebuilt with host-side ASan + UBSan and the CPU tests of the
C ABI are run against that build in a child process that preloads the
sanitizer runtime.  Any sanitizer report fails the test.  CPU only: no
kernel is launched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow

CHECK_LOADED = (
    "import block_sparse_softmax_attn_amd._lib as L; L.get(); "
    "maps = open('/proc/self/maps').read(); "
    "assert L.LIB_PATH in maps and L.LIB_PATH.endswith('/asan/libbsattn.so'), L.LIB_PATH; "
    "import ctypes; ctypes.CDLL(None).__asan_init; print('sanitized library loaded')"
)


def _sanitized_env(log_dir):
    from block_sparse_softmax_attn_amd import build as b
    if not all(os.path.exists(os.path.join(b.BUILD, os.path.basename(s) + ".o")) for s in b.sources()):
        b.build(verbose=False)
    lib = b.build_sanitized(verbose=False)
    rt = b.sanitizer_runtime()
    env = dict(os.environ)
    # the sanitizer runtime has to come first in the preload list
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # reports go to files: pytest's output capture loses what a process that
    # the sanitizer stops has written to stderr
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={log_dir}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log_dir}/ubsan"
    env["BSATTN_LIBRARY"] = lib
    return env


def _reports(log_dir):
    return "".join(open(os.path.join(log_dir, f)).read() for f in sorted(os.listdir(log_dir)))


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    env = _sanitized_env(tmp_path)
    r = subprocess.run([sys.executable, "-c", CHECK_LOADED], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout + r.stderr + _reports(tmp_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_zz_no_alloc.py",
                        "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    reports = _reports(tmp_path)
    assert not reports, reports[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
