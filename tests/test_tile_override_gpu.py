"""The ATTN_TILE and ATTN_W64 tuning overrides (read once per process, so each
setting runs in a child process).  Forcing 128- or 256-row workgroups of 32-row
waves on the bf16 dense and causal forwards gives the same outputs, bit for
bit (ATTN_TILE=128 against ATTN_TILE=256 with ATTN_W64=0); forcing 256 rows
with the 64-row kernel allowed equals the automatic choice; an unknown value
keeps the automatic choice.  The 64-row kernel sums each row's denominator in
another order, so its outputs differ from the 32-row kernels' in the last bits
(its accuracy is checked against the oracle in test_w64_gpu.py)."""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import hashlib, sys, torch
sys.path.insert(0, {root!r})
import block_sparse_softmax_attn_amd as m
import workloads
h = hashlib.sha256()
# automatic shapes: 128 rows (folded: B4 H16 N2048 d64), 128 rows, 256 rows (B1 H32 N8192 d128)
for (B, H, N, d, causal) in [(4, 16, 2048, 64, True), (2, 8, 777, 64, True), (1, 4, 1000, 128, False),
                             (1, 32, 8192, 128, False)]:
    q, k, v = workloads.make_qkv(B, H, N, d, "bf16", 77 + N)
    o, lse = m.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    h.update(o.view(torch.int16).cpu().numpy().tobytes())
    h.update(lse.cpu().numpy().tobytes())
print("digest", h.hexdigest())
"""


def _digest(value, w64=None):
    env = dict(os.environ)
    env.pop("ATTN_TILE", None)
    env.pop("ATTN_W64", None)
    if value is not None:
        env["ATTN_TILE"] = value
    if w64 is not None:
        env["ATTN_W64"] = w64
    print(f"case ATTN_TILE={value} ATTN_W64={w64}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    line = [x for x in r.stdout.splitlines() if x.startswith("digest ")]
    assert line, r.stdout + r.stderr
    return line[-1].split()[1]


def test_forced_workgroup_shapes_give_identical_outputs():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    auto = _digest(None)
    assert _digest("128") == _digest("256", w64="0")
    assert _digest("256") == auto
    assert _digest("not-a-shape") == auto
    assert _digest(None, w64="0") != auto   # the 64-row kernel runs on the N8192 d128 shape
