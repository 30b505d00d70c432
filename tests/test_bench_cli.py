"""The measurement script's contract, on the CPU: one GPU only, no silent
run without a GPU, the CPU baseline is the oracle's own record, and stored HBM
byte counts are used only for the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import pytest
import torch

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_more_or_fewer_than_one_gpu_is_refused(n):
    r = _run("--gpus", n)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the refusal on a machine without a GPU")
def test_no_gpu_is_an_error_not_a_fallback():
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 1 and r.stdout == ""
    assert "needs a ROCm GPU" in r.stderr


def test_unknown_workload_is_refused():
    r = _run("--workload", "no-such-workload")
    assert r.returncode == 2 and "invalid choice" in r.stderr


def test_allowed_pairs_closed_forms():
    dense = workloads.CONFIGS["dense-h32-n8192-d128"]
    assert bench.allowed_pairs_dense(dense) == 32 * 8192 * 8192
    causal = workloads.CONFIGS["causal-b4-h16-n2048-d64"]
    assert bench.allowed_pairs_dense(causal) == 4 * 16 * 2048 * 2049 // 2


def test_cpu_baseline_is_the_oracle_on_whole_heads():
    cfg = workloads.CONFIGS["dense-f32-h1-n256-d64"]
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    rec = bench.cpu_baseline(cfg, q, k, v, budget_s=0.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["sample"].startswith(f"1 of {cfg.B * cfg.H} (batch, head) pairs of {cfg.name}")


def test_stored_traffic_is_used_only_for_the_same_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "fwd_{workload}_traffic.json"))
    assert bench.read_traffic("w") is None                   # nothing stored
    rec = {"kernel_source_sha256": bench.kernel_source_hash(), "traffic_bytes_per_launch": 12345}
    (tmp_path / "fwd_w_traffic.json").write_text(json.dumps(rec))
    assert bench.read_traffic("w") == 12345
    rec["kernel_source_sha256"] = "0" * 64                    # taken on another version of the kernel
    (tmp_path / "fwd_w_traffic.json").write_text(json.dumps(rec))
    assert bench.read_traffic("w") is None


def test_committed_traffic_records_name_their_workloads():
    # profiles/<kernel>_<workload>_traffic.json, <kernel> the one bench.py names for the workload
    prof = os.path.join(ROOT, "profiles")
    seen = 0
    for name in os.listdir(prof):
        if name.endswith("_traffic.json"):
            rec = json.load(open(os.path.join(prof, name)))
            stem = name[:-len("_traffic.json")]
            found = [w for w in workloads.CONFIGS if stem.endswith("_" + w)]
            assert len(found) == 1, name
            cfg = workloads.CONFIGS[found[0]]
            assert stem == bench.fwd_kernel_name(cfg).replace("_kernel", "") + "_" + cfg.name, name
            assert rec["workload"] == cfg.description, name
            assert rec["traffic_bytes_per_launch"] > 0 and len(rec["kernel_source_sha256"]) == 64
            seen += 1
    assert seen >= 4


def test_cpu_baseline_reports_host_cores_and_blas_threads_separately():
    cfg = workloads.CONFIGS["dense-f32-h1-n256-d64"]
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    rec = bench.cpu_baseline(cfg, q, k, v, budget_s=0.0)
    assert rec["cores"] == len(os.sched_getaffinity(0))
    assert rec["blas_threads"] >= 1
    assert rec["rows_per_s"] > 0


def test_cpu_baseline_on_sampled_rows_reports_rows_per_second_and_a_labelled_extrapolation():
    import dataclasses
    cfg = dataclasses.replace(workloads.CONFIGS["causal-h8-n131072-d128"], H=2, N=4096, sample_rows=256)
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    rec = bench.cpu_baseline(cfg, q, k, v, budget_s=0.0)
    assert rec["sample"].startswith("256 sampled query rows of each of 1 of 2 (batch, head) pairs")
    assert rec["extrapolated_all_rows_s"] > 0 and "extrapolation" in rec
    # the rate counts the allowed pairs of the sampled rows only (causal: row r sees r + 1 keys)
    assert rec["value"] > 0


def test_oracle_check_passes_the_oracle_and_catches_a_planted_error():
    import numpy as np
    import oracle
    cfg = workloads.CONFIGS["causal-b4-h16-n2048-d64"]
    import dataclasses
    cfg = dataclasses.replace(cfg, B=1, H=2, N=300)
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, cfg.scale, cfg.causal)
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).float()
    rec = bench.oracle_check(cfg, q, k, v, o, lse, rows_per_head=32)
    assert rec["ok"] and rec["max_abs_dO"] <= 1e-2 and rec["max_abs_dLSE"] <= 1e-3
    rows = workloads.sample_rows(cfg.N, 32, 77 * 1000 + 1)        # the rows checked on head 1
    bad = o.clone()
    bad[0, 1, rows[5], 3] += 0.05
    rec = bench.oracle_check(cfg, q, k, v, bad, lse, rows_per_head=32)
    assert not rec["ok"] and rec["max_abs_dO"] > 0.04
    bad_l = lse.clone()
    bad_l[0, 0, workloads.sample_rows(cfg.N, 32, 77 * 1000)[0]] = float("nan")
    assert not bench.oracle_check(cfg, q, k, v, o, bad_l, rows_per_head=32)["ok"]


def test_executed_tiles_of_causal_runs():
    c2 = workloads.CONFIGS["causal-b4-h16-n2048-d64"]
    assert bench.executed_tiles_128(c2) == 8704        # 64 heads x 16 * 17 / 2
    c5 = workloads.CONFIGS["causal-h8-n131072-d128"]
    assert bench.executed_tiles_128(c5) == 4198400


def test_oracle_check_holds_empty_rows_to_zero_and_minus_inf():
    import dataclasses
    import numpy as np
    import oracle
    cfg = dataclasses.replace(workloads.CONFIGS["sparse-causal-h16-n16300-d128"], H=1, N=640)
    nqb = cfg.N // cfg.block
    rows = [[qb] if qb != 2 else [] for qb in range(nqb)]     # query block 2 lists nothing
    rp, col = workloads.lists_to_csr(rows)
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    o_ref, lse_ref = oracle.attn_fwd_blocksparse(q, k, v, cfg.scale, True, cfg.block, rp, col, 1)
    assert np.isinf(lse_ref[0, 0, 256:384]).all()
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).float()
    check = lambda o_, l_: bench.oracle_check(cfg, q, k, v, o_, l_, rows_per_head=640, mask_lists=(rp, col))["ok"]
    assert check(o, lse)
    bad_l = lse.clone()
    bad_l[0, 0, 300] = float("inf")          # an empty row must give -inf, not +inf
    assert not check(o, bad_l)
    bad_o = o.clone()
    bad_o[0, 0, 300, 7] = 1e-3               # and O exactly 0
    assert not check(bad_o, lse)


def test_algorithmic_bytes():
    # dense: Q, K, V read and O written once (bf16), 4 B of LSE per row
    c3 = workloads.CONFIGS["dense-h32-n8192-d128"]
    assert bench.algorithmic_bytes(c3) == 4 * 32 * 8192 * 128 * 2 + 32 * 8192 * 4
    c1 = workloads.CONFIGS["dense-f32-h1-n256-d64"]
    assert bench.algorithmic_bytes(c1) == 4 * 256 * 64 * 4 + 256 * 4
    # block-sparse: K and V only for the referenced key blocks (the last one partial)
    import dataclasses
    import block_sparse_softmax_attn_amd as m
    cfg = dataclasses.replace(workloads.CONFIGS["sparse-causal-h16-n16300-d128"], H=2, N=300)
    rp, col = workloads.lists_to_csr([[0], [0], [2, 0]])        # block 1 never referenced
    mask = m.blockmask_build(rp, col, 1, 300, 128, True)
    keys = 128 + (300 - 256)
    assert bench.algorithmic_bytes(cfg, mask) == 2 * 2 * 300 * 128 * 2 + 2 * 300 * 4 + 2 * 2 * keys * 128 * 2


def test_vector_floor_closed_form():
    # one millisecond of the softmax's vector work on every SIMD at 2.4 GHz
    scores = round(1024 * 2.4e9 * 1e-3 / bench.VALU_CYCLES_PER_SCORE)
    vf = bench.vector_floor(scores, 2.0)
    assert abs(vf["floor_ms"] - 1.0) < 1e-4 and abs(vf["frac"] - 0.5) < 1e-4
    assert bench.VALU_CYCLES_PER_SCORE == 4.5 * 4 / 64
    assert "issue_floor_ms" not in vf


def test_issue_floor_closed_form():
    # d = 64: 16 MFMAs per 32 x 64 tile of scores, 11 issue cycles each, on top of
    # the vector work; d = 128 twice the MFMAs
    for d, mfma_per_2048 in ((64, 16), (128, 32)):
        per_score = bench.VALU_CYCLES_PER_SCORE + mfma_per_2048 * bench.MFMA_ISSUE_CYCLES / 2048
        scores = round(1024 * 2.4e9 * 1e-3 / per_score)
        vf = bench.vector_floor(scores, 4.0, d)
        assert abs(vf["issue_cycles_per_score"] - per_score) < 1e-5
        assert abs(vf["issue_floor_ms"] - 1.0) < 1e-4 and abs(vf["issue_frac"] - 0.25) < 1e-4
    # the issue floor binds above the matrix work at d = 64, not at d = 128
    assert 0.28125 + 16 * 11 / 2048 > 64 / 256 and 0.28125 + 32 * 11 / 2048 < 128 / 256
