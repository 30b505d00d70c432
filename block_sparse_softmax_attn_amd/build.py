"""Build the gfx950 attention library in-tree: ``python -m block_sparse_softmax_attn_amd.build``.

Compiles every source under ``csrc/`` with hipcc for gfx950 and links
``libbsattn.so`` next to this file.  Always recompiles (object files go to
``_build/`` at the repository root).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsattn.so")

ARCH = "gfx950"
# Packed fp32 VALU forms stay disabled: hipcc may otherwise form them from
# ordinary float code.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


# Per-source flags.  The 64-row forward keeps its O accumulators in AGPRs by
# writing those products as inline assembly; this makes the compiler keep its
# own (score) products in the VGPR form, whose results the softmax reads.
EXTRA = {"fwd_bf16_w64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = shutil.which("hipcc") or os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: a ROCm toolchain is required to build the library")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer, for the CPU-only
# checking build of the argument validation and the block-mask builder.  Each
# flag is scoped to the host pass (device code is compiled as usual).
SANITIZE = [f for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer")
            for f in ("-Xarch_host", flag)]
# the sources holding the host logic that the sanitized build instruments
SANITIZED_SOURCES = ("api.cpp", "blockmask.cpp")
SANITIZED_LIB = os.path.join(BUILD, "asan", "libbsattn.so")


def _compile(src: str, obj_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """A checking build at ``_build/asan/libbsattn.so``: api.cpp and blockmask.cpp
    compiled with host ASan/UBSan, linked with the kernel objects of the normal
    build (which must exist).  It is loaded only by a CPU test, in a process
    that preloads the sanitizer runtime; the product library is never it."""
    out = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out, exist_ok=True)
    objs = []
    for src in sources():
        name = os.path.basename(src)
        if name in SANITIZED_SOURCES:
            objs.append(_compile(src, out, SANITIZE))
        else:
            obj = os.path.join(BUILD, name + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run the normal build first")
            objs.append(obj)
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SANITIZED_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {SANITIZED_LIB}")
    return SANITIZED_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it carries the UBSan handlers)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's shared ASan runtime was not found")
    return path


if __name__ == "__main__":
    build()
