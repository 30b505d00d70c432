"""GPU parity of the d = 128 forward with 64 query rows per wave (the kernel the
library launches for large bf16 dense and causal grids of whole 64-key tiles),
through the C ABI, against the float64 oracle on every row.

The kernel is chosen for grids of at least 1024 256-row query tiles; these
shapes are smaller, so each case runs in a child process with ATTN_TILE=256
(read once per process), which makes the dispatcher treat every grid as large.
Causal cases cover the element mask on the sub-tiles that cross a wave's rows,
sub-tiles wholly past them (computed and masked), and workgroups whose key
range ends at their own last row.
Tile counts 2 to 5 cover the pipeline's prologue, its two-tile loop body, the
single leftover tile and the last two tiles; 16 and 17 tiles cover many trips
of the loop with an even and an odd count; GQA shares K/V heads; growing
logits force the rescale path on most sub-tiles.  The same launches with
ATTN_W64=0 take the 32-row kernel, whose outputs must differ in the last bits
(the denominator is summed in another order): evidence that the 64-row kernel
is the one under test.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import compare, to64

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (B, H, Hkv, N, causal, seed): N a multiple of 64 (2 to 17 tiles of 64 keys)
CASES = [(1, 2, 2, 128, False, 1), (1, 2, 2, 192, False, 2), (1, 3, 3, 256, False, 3), (2, 2, 2, 320, False, 4),
         (1, 2, 2, 1024, False, 5), (1, 1, 1, 1088, False, 6), (1, 4, 2, 512, False, 7),
         (1, 2, 2, 128, True, 11), (1, 2, 2, 320, True, 12), (2, 2, 2, 576, True, 13), (1, 4, 2, 1088, True, 14),
         (1, 3, 3, 704, True, 15)]

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
import block_sparse_softmax_attn_amd as m
import workloads
out = {{}}
for (B, H, Hkv, N, causal, seed) in {cases!r}:
    g = torch.Generator().manual_seed(1000 + seed)
    q = torch.randn((B, H, N, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, 128), generator=g).to(torch.bfloat16)
    print("case", B, H, Hkv, N, causal, flush=True)
    o, lse = m.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    key = f"{{B}}_{{H}}_{{Hkv}}_{{N}}_{{int(causal)}}"
    out["o_" + key] = o.float().cpu().numpy()
    out["lse_" + key] = lse.cpu().numpy()
# growing logits: key j = (j + 1) k0, so most sub-tiles raise the row's reference value
g = torch.Generator().manual_seed(4242)
q = torch.randn((1, 2, 768, 128), generator=g).to(torch.bfloat16)
k0 = torch.randn((1, 2, 1, 128), generator=g)
v = (0.25 * torch.randn((1, 2, 768, 128), generator=g)).to(torch.bfloat16)
growth = torch.arange(1, 769, dtype=torch.float32).view(1, 1, 768, 1)
k = (k0 * growth).to(torch.bfloat16)
print("case growing logits", flush=True)
o, lse = m.attn_fwd(q.cuda(), k.cuda(), v.cuda())
torch.cuda.synchronize()
out["o_grow"] = o.float().cpu().numpy()
out["lse_grow"] = lse.cpu().numpy()
out["q_grow"] = q.float().numpy(); out["k_grow"] = k.float().numpy(); out["v_grow"] = v.float().numpy()
np.savez({path!r}, **out)
print("done", flush=True)
"""


def _run(tmp_path, w64):
    path = str(tmp_path / f"w64_{w64}.npz")
    env = dict(os.environ)
    env["ATTN_TILE"] = "256"
    env.pop("ATTN_W64", None)
    if w64 is not None:
        env["ATTN_W64"] = w64
    print(f"child ATTN_TILE=256 ATTN_W64={w64}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, cases=CASES, path=path)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return np.load(path)


@pytest.fixture(scope="module")
def outputs(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    tmp = tmp_path_factory.mktemp("w64")
    return _run(tmp, None), _run(tmp, "0")


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}{'causal' if c[4] else 'dense'}"
                                              for c in CASES])
def test_w64_matches_oracle(outputs, case):
    got, _ = outputs
    B, H, Hkv, N, causal, seed = case
    g = torch.Generator().manual_seed(1000 + seed)
    q = torch.randn((B, H, N, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, 128), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    if Hkv == H:
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    else:
        o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, scale, causal)
    key = f"{B}_{H}_{Hkv}_{N}_{int(causal)}"
    do, dl = compare(got["o_" + key].astype(np.float64), got["lse_" + key].astype(np.float64), o_ref, lse_ref,
                     "bf16", f"w64 {key}")
    print(f"w64 {key}: max|dO| {do:.3e} max|dLSE| {dl:.3e}", flush=True)


def test_w64_growing_logits(outputs):
    got, _ = outputs
    q, k, v = got["q_grow"], got["k_grow"], got["v_grow"]
    o_ref, lse_ref = oracle.attn_fwd(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                     1.0 / math.sqrt(128), False)
    assert np.max(np.abs(v)) <= 1.5   # |V| <= ~1: the fixed N(0,1) bounds hold (P rounding, O's half ulp)
    do = float(np.max(np.abs(got["o_grow"].astype(np.float64) - o_ref)))
    dl = float(np.max(np.abs(got["lse_grow"].astype(np.float64) - lse_ref)))
    print(f"w64 growing logits: max|dO| {do:.3e} max|dLSE| {dl:.3e}", flush=True)
    assert do <= 1e-2 and dl <= 1e-3


def test_w64_is_the_kernel_under_test(outputs):
    w64, w32 = outputs
    differs = any(not np.array_equal(w64[name], w32[name]) for name in w64.files if name.startswith("lse_"))
    assert differs, "ATTN_W64=0 gave bitwise the same outputs: the 64-row kernel did not run"
