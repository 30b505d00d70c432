"""The backward entry point that allocates nothing (attn_bwd_noalloc) against
attn_bwd, through the C ABI: two calls in a row, the second on smaller
inputs, must give the same gradients bit for bit; sizes past the library's
fixed scratch are refused before any launch (checked on the CPU)."""
import ctypes
import math

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")


def _lib():
    import block_sparse_softmax_attn_amd as m
    return m


def test_noalloc_refuses_sizes_past_its_scratch_without_a_gpu():
    from block_sparse_softmax_attn_amd import _lib as L
    lib = L.get()
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: refused before any launch
    B, H, N, d = 1, 64, 1 << 20, 128  # statistics of 64 heads of 2^20 rows: 512 MiB > the scratch
    need = lib.attn_bwd_workspace_bytes(B, H, N, d, L.ATTN_BF16)
    assert need > L.ATTN_NOALLOC_SCRATCH_BYTES
    st = lib.attn_bwd_noalloc(*([fake] * 9), B, H, N, d, L.ATTN_BF16, ctypes.c_float(0.088), 1, None)
    assert st == L.ATTN_ECAPACITY
    # the other argument checks still come first
    st = lib.attn_bwd_noalloc(*([fake] * 9), B, H, N, 96, L.ATTN_BF16, ctypes.c_float(0.088), 1, None)
    assert st == L.ATTN_EUNSUPPORTED
    st = lib.attn_bwd_noalloc(*([fake] * 9), B, H, N, d, L.ATTN_BF16, ctypes.c_float(-1.0), 1, None)
    assert st == L.ATTN_EINVAL


@pytest.mark.gpu
def test_noalloc_backward_equals_attn_bwd_twice_second_smaller():
    m = _lib()
    dev = torch.device("cuda:0")
    for (B, H, N, d, causal, seed) in ((2, 4, 1000, 128, True, 31), (1, 2, 300, 64, False, 32)):
        print(f"case noalloc B{B} H{H} N{N} d{d} causal={causal}", flush=True)
        q, k, v = (t.to(dev) for t in workloads.make_qkv(B, H, N, d, "bf16", seed=seed))
        do = workloads.make_grad(B, H, N, d, seed=seed + 100).to(dev)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        o, lse = m.attn_fwd(q, k, v, scale=scale, causal=causal)
        ref = m.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
        grads = tuple(torch.full_like(q if i == 0 else k, float("nan")) for i in range(3))
        got = m.attn_bwd_noalloc(q, k, v, o, lse, do, scale=scale, causal=causal,
                                 dq=grads[0], dk=grads[1], dv=grads[2])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs from attn_bwd for B{B} H{H} N{N} d{d}"
