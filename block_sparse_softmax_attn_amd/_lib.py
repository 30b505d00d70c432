"""ctypes binding of ``libbsattn.so`` (the C ABI in ``include/bsattn.h``).

Argument marshalling only: every step of the attention forward runs in the HIP
kernels behind the C ABI.  The library is loaded on first use; if it has not
been built, that use raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# BSATTN_LIBRARY names another build of the same library (the host-sanitized
# checking build); by default the in-tree one is loaded.
LIB_PATH = os.environ.get("BSATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libbsattn.so")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_ECAPACITY = -3
ATTN_EHIP = -4
ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_FLAG_DIAGONAL = 1
ATTN_FLAG_PARTIAL = 2
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20   # the library's fixed scratch for attn_bwd_noalloc, per GPU

EXPORTED = ("attn_status_string", "attn_prepared_v_bytes", "attn_fwd", "attn_blockmask_build",
            "attn_fwd_blocksparse", "attn_prepare_v", "attn_fwd_prepared", "attn_fwd_blocksparse_prepared",
            "attn_bwd_workspace_bytes", "attn_bwd", "attn_blockmask_transpose", "attn_bwd_blocksparse",
            "attn_bwd_blocksparse_workspace_bytes",
            "attn_fwd_splitkv_workspace_bytes", "attn_fwd_splitkv", "attn_fwd_block", "attn_merge", "attn_fwd_gqa", "attn_fwd_blocksparse_gqa",
            "attn_bwd_gqa_workspace_bytes", "attn_bwd_gqa", "attn_bwd_blocksparse_gqa",
            "attn_select_meanpool_nnz", "attn_select_meanpool_workspace_bytes", "attn_select_meanpool",
            "attn_bwd_noalloc")


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status} ({text})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_softmax_attn_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_prepared_v_bytes.restype = i64
    lib.attn_prepared_v_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_fwd.restype = i32
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.attn_blockmask_build.restype = i32
    lib.attn_blockmask_build.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, vp, i64, vp, vp, vp]
    lib.attn_fwd_blocksparse.restype = i32
    lib.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, i64,
                                         vp, vp, vp, i64, i64, vp]
    lib.attn_prepare_v.restype = i32
    lib.attn_prepare_v.argtypes = [vp, i64, i64, i64, i64, i32, vp, i64, vp]
    lib.attn_fwd_prepared.restype = i32
    lib.attn_fwd_prepared.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, vp, i64, vp]
    lib.attn_fwd_blocksparse_prepared.restype = i32
    lib.attn_fwd_blocksparse_prepared.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, i64,
                                                  vp, vp, vp, i64, i64, vp, i64, vp]
    lib.attn_bwd_workspace_bytes.restype = i64
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_bwd.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, vp, i64, vp]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.attn_blockmask_transpose.restype = i32
    lib.attn_blockmask_transpose.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64]
    lib.attn_bwd_blocksparse_workspace_bytes.restype = i64
    lib.attn_bwd_blocksparse_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i64, vp, i64]
    lib.attn_bwd_blocksparse.restype = i32
    lib.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, i64,
                                         vp, vp, vp, i64, vp, vp, i64, vp, i64, vp]
    lib.attn_fwd_splitkv_workspace_bytes.restype = i64
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i64]
    lib.attn_fwd_splitkv.restype = i32
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, i64, vp, i64, vp]
    lib.attn_fwd_block.restype = i32
    lib.attn_fwd_block.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, i64, i64, vp]
    lib.attn_merge.restype = i32
    lib.attn_merge.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, i32, vp]
    lib.attn_fwd_gqa.restype = i32
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.attn_fwd_blocksparse_gqa.restype = i32
    lib.attn_fwd_blocksparse_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, i64,
                                             vp, vp, vp, i64, i64, vp]
    lib.attn_bwd_gqa_workspace_bytes.restype = i64
    lib.attn_bwd_gqa_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.attn_bwd_gqa.restype = i32
    lib.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, vp, i64,
                                 vp]
    lib.attn_bwd_blocksparse_gqa.restype = i32
    lib.attn_bwd_blocksparse_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32,
                                             i32, i64, vp, vp, vp, i64, vp, vp, i64, vp, i64, vp]
    lib.attn_select_meanpool_nnz.restype = i64
    lib.attn_select_meanpool_nnz.argtypes = [i64, i64, i64, i64, i32, i64]
    lib.attn_select_meanpool_workspace_bytes.restype = i64
    lib.attn_select_meanpool_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.attn_select_meanpool.restype = i32
    lib.attn_select_meanpool.argtypes = [vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, i64, i64, i32, vp, vp, vp,
                                         i64, vp, i64, vp]
    return lib


_LIB = None


def get() -> ctypes.CDLL:
    """The loaded library (loaded once; raises ImportError if it is not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def status_string(status: int) -> str:
    return get().attn_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(fn, status, status_string(status))
