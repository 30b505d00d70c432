"""Fused softmax attention (dense, causal, block-sparse), forward and backward, for AMD MI355X.

Thin Python layer over the C ABI of ``libbsattn.so``: it checks tensors,
passes raw device pointers and the current HIP stream, and returns the
outputs.  PyTorch only provides device memory and streams; the arithmetic runs
in the gfx950 kernels.

    o, lse = attn_fwd(q, k, v, scale=None, causal=False)
    meta   = blockmask_build(raw_row_ptr, raw_col, meta_heads, N, block, causal)
    o, lse = attn_fwd_blocksparse(q, k, v, meta, causal=True)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=False)
    dq, dk, dv = attn_bwd_blocksparse(q, k, v, o, lse, do, meta)
    o, lse = attn_fwd_splitkv(q, k, v, num_splits=4)
    o_b, lse_b = attn_fwd_block(q_rows, k_blk, v_blk, q_offset=..., k_offset=...)
    o, lse = attn_merge(o_parts, lse_parts)

Operator ("Exact Blocks, Rings, and Sparsity", sections 1, 2 and 5;
"block-sparse attention patterns"): O = softmax(scale * Q K^T) V over the
allowed pairs, LSE = log-sum-exp of the scaled logits (natural log); rows with
no allowed key give O = 0 and LSE = -inf.  The backward ("Exact Blocks,
Rings, and Sparsity", section 3) returns dQ, dK, dV for an upstream gradient
dO, rebuilding P from LSE (bfloat16 only).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import numpy as np

from ._lib import (ATTN_BF16, ATTN_ECAPACITY, ATTN_F32, ATTN_FLAG_DIAGONAL, ATTN_FLAG_PARTIAL,
                   ATTN_NOALLOC_SCRATCH_BYTES, ATTN_OK, AttnError, LIB_PATH, check, get as _get_lib, status_string)

__all__ = ["attn_fwd", "attn_fwd_blocksparse", "blockmask_build", "prepared_v_bytes", "prepare_v", "attn_fwd_prepared",
           "attn_fwd_blocksparse_prepared", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_blocksparse", "bwd_workspace_bytes",
           "bwd_blocksparse_workspace_bytes",
           "attn_fwd_splitkv", "attn_fwd_block", "attn_merge", "select_meanpool", "DeviceBlockMask",
           "BlockMask", "AttnError", "LIB_PATH",
           "status_string", "ATTN_FLAG_DIAGONAL", "ATTN_FLAG_PARTIAL", "ATTN_NOALLOC_SCRATCH_BYTES"]


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _check_qkv(q, k, v):
    """q [B, H, N, d]; k, v [B, Hkv, N, d] with H a multiple of Hkv (Hkv < H is
    grouped-query attention)."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:] or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise ValueError("k, v must be [B, Hkv, N, d] with H a multiple of Hkv")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or len({q.device, k.device, v.device}) != 1:
        raise ValueError("q, k, v must live on one GPU")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")


def _outputs(q, out, lse):
    import torch
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must match q in shape, dtype, device and be contiguous")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    return out, lse


def prepared_v_bytes(B: int, H: int, N: int, d: int) -> int:
    """Bytes of the V^T buffer prepare_v writes (bf16) for these sizes."""
    n = int(_get_lib().attn_prepared_v_bytes(int(B), int(H), int(N), int(d), ATTN_BF16))
    if n < 0:
        raise ValueError("sizes not supported")
    return n


def _vt_buffer(B, H, N, d, dev, vt):
    """A V^T buffer for B*H heads (allocated from torch's caching allocator
    when ``vt`` is None)."""
    import torch
    need = prepared_v_bytes(B, H, N, d)
    if vt is None:
        vt = torch.empty(need, dtype=torch.uint8, device=dev)
    if vt.device != dev or not vt.is_contiguous() or vt.numel() * vt.element_size() < need:
        raise ValueError(f"the V^T buffer must be a contiguous buffer of at least {need} bytes on the inputs' device")
    return vt, vt.numel() * vt.element_size()


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def attn_fwd(q, k, v, scale: Optional[float] = None, causal: bool = False, out=None, lse=None):
    """Dense or causal attention forward; returns (O in q's dtype, LSE fp32 [B,H,N])."""
    import torch
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    with torch.cuda.device(q.device):
        if Hkv == H:
            st = _get_lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, _dtype_code(q), ctypes.c_float(scale), int(bool(causal)),
                                     _stream(q.device))
        else:
            st = _get_lib().attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                         B, H, Hkv, N, d, _dtype_code(q), ctypes.c_float(scale), int(bool(causal)),
                                         _stream(q.device))
    check("attn_fwd", st)
    return out, lse


@dataclasses.dataclass
class BlockMask:
    """Canonical block-sparse metadata (host arrays) and its pair counts."""
    N: int
    block: int
    causal: bool
    meta_heads: int
    row_ptr: np.ndarray              # int32 [meta_heads * nqb + 1]
    col: np.ndarray                  # int32 [nnz]
    flags: np.ndarray                # uint8 [nnz]
    allowed_pairs: np.ndarray        # int64 [meta_heads]
    executed_tile_pairs: np.ndarray  # int64 [meta_heads]
    _device: dict = dataclasses.field(default_factory=dict, repr=False)

    @property
    def nnz(self) -> int:
        return int(self.col.size)

    def to_device(self, device):
        """Device copies (row_ptr, col, flags), cached per device."""
        import torch
        key = str(device)
        if key not in self._device:
            col = self.col if self.col.size else np.zeros(1, np.int32)
            flags = self.flags if self.flags.size else np.zeros(1, np.uint8)
            self._device[key] = tuple(torch.from_numpy(np.ascontiguousarray(x)).to(device)
                                      for x in (self.row_ptr, col, flags))
        return self._device[key]

    def transposed(self):
        """Host (t_row_ptr, t_col): for each key block, the query blocks that
        list it, in increasing order (computed once, in the library)."""
        if "_t" not in self._device:
            nb = -(-self.N // self.block)
            t_row_ptr = np.zeros(self.meta_heads * nb + 1, dtype=np.int32)
            t_col = np.zeros(max(self.nnz, 1), dtype=np.int32)
            col = self.col if self.col.size else np.zeros(1, np.int32)
            ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
            st = _get_lib().attn_blockmask_transpose(ptr(self.row_ptr), ptr(col), self.meta_heads, self.N,
                                                     self.block, ptr(t_row_ptr), ptr(t_col), t_col.size)
            check("attn_blockmask_transpose", st)
            self._device["_t"] = (t_row_ptr, t_col)
        return self._device["_t"]

    def transposed_to_device(self, device):
        """Device copies of ``transposed()``, cached per device."""
        import torch
        key = "_t:" + str(device)
        if key not in self._device:
            self._device[key] = tuple(torch.from_numpy(x).to(device) for x in self.transposed())
        return self._device[key]


def blockmask_build(raw_row_ptr, raw_col, meta_heads: int, N: int, block: int, causal: bool) -> BlockMask:
    """Canonicalise raw per-query-block key-block lists (host, in the library)."""
    rp = np.ascontiguousarray(np.asarray(raw_row_ptr, dtype=np.int32))
    rc = np.ascontiguousarray(np.asarray(raw_col, dtype=np.int32))
    nqb = -(-int(N) // int(block)) if block > 0 else 0
    if rp.shape != (int(meta_heads) * nqb + 1,):
        raise ValueError("raw_row_ptr must hold meta_heads * ceil(N / block) + 1 offsets")
    cap = max(int(rc.size), 1)
    row_ptr = np.zeros(rp.size, dtype=np.int32)
    col = np.zeros(cap, dtype=np.int32)
    flags = np.zeros(cap, dtype=np.uint8)
    nnz = np.zeros(1, dtype=np.int64)
    allowed = np.zeros(max(int(meta_heads), 1), dtype=np.int64)
    executed = np.zeros(max(int(meta_heads), 1), dtype=np.int64)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = _get_lib().attn_blockmask_build(ptr(rp), ptr(rc) if rc.size else None, int(meta_heads), int(N), int(block),
                                  int(bool(causal)), ptr(row_ptr), ptr(col), ptr(flags), cap, ptr(nnz),
                                  ptr(allowed), ptr(executed))
    check("attn_blockmask_build", st)
    n = int(nnz[0])
    return BlockMask(int(N), int(block), bool(causal), int(meta_heads), row_ptr, col[:n].copy(),
                     flags[:n].copy(), allowed[:meta_heads].copy(), executed[:meta_heads].copy())


def attn_fwd_blocksparse(q, k, v, mask: BlockMask, scale: Optional[float] = None, causal: Optional[bool] = None,
                         out=None, lse=None):
    """Block-sparse attention forward, renormalised over the allowed pairs."""
    import torch
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if mask.N != N:
        raise ValueError(f"mask was built for N={mask.N}, inputs have N={N}")
    causal = mask.causal if causal is None else bool(causal)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    row_ptr, col, flags = mask.to_device(q.device)
    Hkv = k.shape[1]
    with torch.cuda.device(q.device):
        if Hkv == H:
            st = _get_lib().attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                 lse.data_ptr(), B, H, N, d, _dtype_code(q), ctypes.c_float(scale),
                                                 int(causal), mask.block, row_ptr.data_ptr(), col.data_ptr(),
                                                 flags.data_ptr(), mask.nnz, mask.meta_heads, _stream(q.device))
        else:
            st = _get_lib().attn_fwd_blocksparse_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                     lse.data_ptr(), B, H, Hkv, N, d, _dtype_code(q),
                                                     ctypes.c_float(scale), int(causal), mask.block,
                                                     row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(), mask.nnz,
                                                     mask.meta_heads, _stream(q.device))
    check("attn_fwd_blocksparse", st)
    return out, lse


def prepare_v(v, vt=None):
    """bf16 only: V transposed into a V^T buffer for attn_fwd_prepared /
    attn_fwd_blocksparse_prepared (returns the buffer)."""
    import torch
    if v.dim() != 4 or not v.is_cuda or not v.is_contiguous() or v.dtype != torch.bfloat16:
        raise ValueError("v must be a contiguous bfloat16 [B, H, N, d] tensor on a GPU")
    B, H, N, d = v.shape
    vt, vt_bytes = _vt_buffer(B, H, N, d, v.device, vt)
    with torch.cuda.device(v.device):
        st = _get_lib().attn_prepare_v(v.data_ptr(), B, H, N, d, ATTN_BF16, vt.data_ptr(), vt_bytes, _stream(v.device))
    check("attn_prepare_v", st)
    return vt


def attn_fwd_prepared(q, k, vt, scale: Optional[float] = None, causal: bool = False, out=None, lse=None):
    """attn_fwd with V^T taken from a buffer filled by prepare_v (bf16)."""
    import torch
    _check_qkv(q, k, k)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    vt, vt_bytes = _vt_buffer(B, H, N, d, q.device, vt)
    with torch.cuda.device(q.device):
        st = _get_lib().attn_fwd_prepared(q.data_ptr(), k.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                                          _dtype_code(q), ctypes.c_float(scale), int(bool(causal)), vt.data_ptr(),
                                          vt_bytes, _stream(q.device))
    check("attn_fwd_prepared", st)
    return out, lse


def attn_fwd_blocksparse_prepared(q, k, vt, mask: BlockMask, scale: Optional[float] = None,
                                  causal: Optional[bool] = None, out=None, lse=None):
    """attn_fwd_blocksparse with V^T taken from a buffer filled by prepare_v (bf16)."""
    import torch
    _check_qkv(q, k, k)
    B, H, N, d = q.shape
    if mask.N != N:
        raise ValueError(f"mask was built for N={mask.N}, inputs have N={N}")
    causal = mask.causal if causal is None else bool(causal)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    row_ptr, col, flags = mask.to_device(q.device)
    vt, vt_bytes = _vt_buffer(B, H, N, d, q.device, vt)
    with torch.cuda.device(q.device):
        st = _get_lib().attn_fwd_blocksparse_prepared(
            q.data_ptr(), k.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, _dtype_code(q),
            ctypes.c_float(scale), int(causal), mask.block, row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(),
            mask.nnz, mask.meta_heads, vt.data_ptr(), vt_bytes, _stream(q.device))
    check("attn_fwd_blocksparse_prepared", st)
    return out, lse


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def bwd_workspace_bytes(B: int, H: int, N: int, d: int, Hkv: Optional[int] = None) -> int:
    """Device workspace (bytes) the bf16 backward needs for these sizes
    (Hkv key/value heads; default H)."""
    Hkv = H if Hkv is None else int(Hkv)
    n = int(_get_lib().attn_bwd_gqa_workspace_bytes(int(B), int(H), Hkv, int(N), int(d), ATTN_BF16))
    if n < 0:
        raise ValueError("sizes not supported by the backward")
    return n


def _bwd_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace, need=None, alloc=None):
    """Checked gradient outputs and workspace: a given workspace needs ``need``
    bytes; one is allocated (``alloc`` bytes, default ``need``) when none is
    given, except for ``need == 0``, where no workspace is returned."""
    import torch
    _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise TypeError("the backward takes bfloat16 tensors")
    B, H, N, d = q.shape
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype, device and be contiguous")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    grads = []
    for g, like in ((dq, q), (dk, k), (dv, v)):
        g = torch.empty_like(like) if g is None else g
        if g.shape != like.shape or g.dtype != q.dtype or not g.is_contiguous() or g.device != q.device:
            raise ValueError("gradient outputs must match q (dq) or k, v (dk, dv) and be contiguous")
        grads.append(g)
    if need is None:
        need = int(_get_lib().attn_bwd_gqa_workspace_bytes(B, H, k.shape[1], N, d, ATTN_BF16))
    if need < 0:
        raise ValueError("sizes not supported by the backward")
    if workspace is None and need == 0 and not alloc:
        return grads, None, 0   # the call takes no workspace
    if workspace is None:
        workspace = torch.empty(max(need, alloc or 0), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a contiguous buffer of at least {need} bytes on the inputs' device")
    return grads, workspace, workspace.numel() * workspace.element_size()


def attn_bwd(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False,
             dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dQ, dK, dV) of attn_fwd for the upstream gradient ``dout``;
    ``o`` and ``lse`` are the forward's outputs for the same inputs (bf16)."""
    import torch
    B, H, N, d = q.shape
    (dq, dk, dv), ws, ws_bytes = _bwd_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    Hkv = k.shape[1]
    with torch.cuda.device(q.device):
        st = _get_lib().attn_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                                     ATTN_BF16, ctypes.c_float(scale), int(bool(causal)), ws.data_ptr(), ws_bytes,
                                     _stream(q.device)) if Hkv != H else \
            _get_lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, ATTN_BF16,
                                ctypes.c_float(scale), int(bool(causal)), ws.data_ptr(), ws_bytes, _stream(q.device))
    check("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False,
                     dq=None, dk=None, dv=None):
    """attn_bwd without a workspace: the library keeps the row statistics in
    its own fixed per-GPU array (for callers that cannot allocate; pass dq, dk,
    dv to allocate nothing here either).  Calls that overlap on one GPU race."""
    import torch
    B, H, N, d = q.shape
    if k.shape[1] != H:
        raise ValueError("attn_bwd_noalloc takes as many key/value heads as query heads")
    (dq, dk, dv), _, _ = _bwd_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace=None, need=0)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        st = _get_lib().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                                         ATTN_BF16, ctypes.c_float(scale), int(bool(causal)), _stream(q.device))
    check("attn_bwd_noalloc", st)
    return dq, dk, dv


def bwd_blocksparse_workspace_bytes(B: int, H: int, N: int, d: int, mask, Hkv: Optional[int] = None) -> int:
    """Device workspace (bytes) the bf16 block-sparse backward uses for this
    mask, including the partial sums of split key-block lists."""
    Hkv = H if Hkv is None else int(Hkv)
    t_row_ptr = np.ascontiguousarray(mask.transposed()[0], dtype=np.int32)
    n = int(_get_lib().attn_bwd_blocksparse_workspace_bytes(int(B), int(H), Hkv, int(N), int(d), ATTN_BF16,
                                                           int(mask.block), t_row_ptr.ctypes.data_as(ctypes.c_void_p),
                                                           int(mask.meta_heads)))
    if n < 0:
        raise ValueError("sizes or metadata not supported by the block-sparse backward")
    return n


def attn_bwd_blocksparse(q, k, v, o, lse, dout, mask: BlockMask, scale: Optional[float] = None,
                         causal: Optional[bool] = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of attn_fwd_blocksparse (bf16)."""
    import torch
    B, H, N, d = q.shape
    if mask.N != N:
        raise ValueError(f"mask was built for N={mask.N}, inputs have N={N}")
    # a smaller workspace than the full size (down to the minimum) turns the
    # split of long key-block lists off
    full = bwd_blocksparse_workspace_bytes(B, H, N, d, mask, Hkv=k.shape[1])
    least = int(_get_lib().attn_bwd_blocksparse_workspace_bytes(B, H, k.shape[1], N, d, ATTN_BF16, int(mask.block),
                                                               None, int(mask.meta_heads)))
    (dq, dk, dv), ws, ws_bytes = _bwd_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace, least, full)
    causal = mask.causal if causal is None else bool(causal)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    row_ptr, col, flags = mask.to_device(q.device)
    t_row_ptr, t_col = mask.transposed_to_device(q.device)
    Hkv = k.shape[1]
    with torch.cuda.device(q.device):
        st = _get_lib().attn_bwd_blocksparse_gqa(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, ATTN_BF16, ctypes.c_float(scale),
            int(causal), mask.block, row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(), mask.nnz,
            t_row_ptr.data_ptr(), t_col.data_ptr(), mask.meta_heads, ws.data_ptr(), ws_bytes, _stream(q.device))
    check("attn_bwd_blocksparse", st)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# key splits, ring steps and the partial-state merge (bf16 inputs)
# ---------------------------------------------------------------------------

def _ws_buffer(dev, need, workspace, align=256):
    import torch
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if (workspace.device != dev or not workspace.is_contiguous()
            or workspace.numel() * workspace.element_size() < need or workspace.data_ptr() % align):
        raise ValueError(f"workspace must be a contiguous, {align}-byte aligned buffer of at least {need} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def attn_fwd_splitkv(q, k, v, scale: Optional[float] = None, causal: bool = False, num_splits: int = 4,
                     out=None, lse=None, workspace=None):
    """attn_fwd over ``num_splits`` key ranges launched together, then merged."""
    import torch
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    need = int(_get_lib().attn_fwd_splitkv_workspace_bytes(B, H, N, d, _dtype_code(q), int(num_splits)))
    if need < 0:
        raise ValueError("sizes, dtype or num_splits not supported by the split-key forward")
    ws, ws_bytes = _ws_buffer(q.device, need, workspace)
    with torch.cuda.device(q.device):
        st = _get_lib().attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                         B, H, N, d, _dtype_code(q), ctypes.c_float(scale), int(bool(causal)),
                                         int(num_splits), ws.data_ptr(), ws_bytes, _stream(q.device))
    check("attn_fwd_splitkv", st)
    return out, lse


def attn_fwd_block(q, k, v, scale: Optional[float] = None, causal: bool = False, q_offset: int = 0,
                   k_offset: int = 0, o_part=None, lse_part=None):
    """One ring step: fp32 partial state (O_b, LSE_b) of the rows of ``q``
    (global positions q_offset + i) against the key/value block ``k``, ``v``
    (global positions k_offset + j)."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or len({q.device, k.device, v.device}) != 1:
        raise ValueError("q, k, v must live on one GPU")
    if not all(t.dtype == torch.bfloat16 and t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must be contiguous bfloat16")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if o_part is None:
        o_part = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = _get_lib().attn_fwd_block(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                       lse_part.data_ptr(), B, H, Nq, Nk, d, ATTN_BF16, ctypes.c_float(scale),
                                       int(bool(causal)), int(q_offset), int(k_offset), _stream(q.device))
    check("attn_fwd_block", st)
    return o_part, lse_part


def attn_merge(o_parts, lse_parts, out_dtype=None, out=None, lse=None):
    """Merge partial states: o_parts fp32 [S, B, H, N, d], lse_parts fp32
    [S, B, H, N] -> (O of out_dtype (float32 default), LSE)."""
    import torch
    if o_parts.dim() != 5 or lse_parts.shape != o_parts.shape[:4]:
        raise ValueError("o_parts must be [S, B, H, N, d] and lse_parts [S, B, H, N]")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partial states are float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("partial states must be contiguous")
    S, B, H, N, d = o_parts.shape
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    code = ATTN_BF16 if out_dtype == torch.bfloat16 else ATTN_F32
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    with torch.cuda.device(o_parts.device):
        st = _get_lib().attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, B, H, N, d, out.data_ptr(),
                                   lse.data_ptr(), code, _stream(o_parts.device))
    check("attn_merge", st)
    return out, lse


# ---------------------------------------------------------------------------
# mean-pooled block selector (metadata built on the device)
# ---------------------------------------------------------------------------

class DeviceBlockMask:
    """Canonical block-sparse metadata that lives on the device (as written by
    the selector): one pattern per (batch, head).  Usable wherever a BlockMask
    is; host copies and pair counts are made on first use."""

    def __init__(self, N, block, causal, meta_heads, row_ptr, col, flags):
        self.N, self.block, self.causal, self.meta_heads = int(N), int(block), bool(causal), int(meta_heads)
        self._dev = (row_ptr, col, flags)
        self._host = None
        self._counts = None
        self._t = {}

    @property
    def nnz(self) -> int:
        return int(self._dev[1].numel())

    def to_device(self, device):
        if self._dev[0].device != device:
            raise ValueError("the selector's metadata lives on another device")
        return self._dev

    def host(self) -> "BlockMask":
        """A host BlockMask with the same lists (copies from the device)."""
        if self._host is None:
            rp, col, fl = (t.cpu().numpy() for t in self._dev)
            counts = blockmask_build(rp, col, self.meta_heads, self.N, self.block, self.causal)
            self._host = counts
        return self._host

    @property
    def row_ptr(self):
        return self.host().row_ptr

    @property
    def col(self):
        return self.host().col

    @property
    def flags(self):
        return self.host().flags

    @property
    def allowed_pairs(self):
        return self.host().allowed_pairs

    @property
    def executed_tile_pairs(self):
        return self.host().executed_tile_pairs

    def transposed(self):
        return self.host().transposed()

    def transposed_to_device(self, device):
        key = str(device)
        if key not in self._t:
            import torch
            self._t[key] = tuple(torch.from_numpy(x).to(device) for x in self.transposed())
        return self._t[key]


def select_meanpool(q, k, block: int, topk: int, causal: bool = False, scale: Optional[float] = None,
                    share_groups: bool = False, workspace=None) -> DeviceBlockMask:
    """Top-k key blocks per query block by mean-pooled tile score, on the device."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError("q must be [B, H, N, d] and k [B, Hkv, N, d]")
    if not (q.is_contiguous() and k.is_contiguous()) or q.device != k.device or not q.is_cuda:
        raise ValueError("q and k must be contiguous and on one GPU")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = _get_lib()
    nnz = int(lib.attn_select_meanpool_nnz(B, H, N, int(block), int(bool(causal)), int(topk)))
    need = int(lib.attn_select_meanpool_workspace_bytes(B, H, Hkv, N, d, int(block)))
    if nnz < 0 or need < 0:
        raise ValueError("sizes, block or topk not supported by the selector")
    nb = -(-N // int(block))
    row_ptr = torch.empty(B * H * nb + 1, dtype=torch.int32, device=q.device)
    col = torch.empty(max(nnz, 1), dtype=torch.int32, device=q.device)
    flags = torch.empty(max(nnz, 1), dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        st = lib.attn_select_meanpool(q.data_ptr(), k.data_ptr(), B, H, Hkv, N, d, _dtype_code(q),
                                      ctypes.c_float(scale), int(bool(causal)), int(block), int(topk),
                                      int(bool(share_groups)), row_ptr.data_ptr(), col.data_ptr(), flags.data_ptr(),
                                      nnz, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(q.device))
    check("attn_select_meanpool", st)
    return DeviceBlockMask(N, block, causal, B * H, row_ptr, col[:nnz], flags[:nnz])
