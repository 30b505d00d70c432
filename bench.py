"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense-h32-n8192-d128] [--all]

A step is one pass of the hot path over one batch of synthetic N(0,1) input
already resident in HBM: one attn_fwd (dense, causal) or
attn_fwd_blocksparse call, i.e. host validation and the single launch of the
fused kernel, which reads Q, K and V in place.  The default workload is the
dense non-causal d=128 case (B=1 H=32 N=8192), the one the throughput target
is stated on.  Prints ONE JSON line (--all: one line per workload, the
fp32 one included):

  value    allowed-pair TFLOP/s over the K timed steps (4*d flops per allowed
           query-key pair: the QK^T and PV contractions), wall clock between
           two device synchronisations;
  timing   the fused kernel's duration per launch (HIP events on the launch
           stream around every EVENT_STRIDE-th timed launch: an event pair
           around every launch adds about 6 us to a 45 us step): mean, median
           and min over those launches;
  roofline the fused kernel against the MFMA peak of its dtype: achieved =
           flops per launch / mean launch duration; traffic = HBM bytes per
           launch from rocprofv3 FETCH_SIZE and WRITE_SIZE counters
           (calibrated on a plain copy), read from profiles/ and reported only
           while the kernel source is unchanged;
  config   the workload; for causal and block-sparse runs also the executed
           work in b x b tiles (b = 128) and its rate;
  check    after the timed steps, max|dO| and max|dLSE| of the timed output
           against the float64 oracle on seeded query rows of every head,
           with the tolerances (bf16 1e-2 / 1e-3, fp32 1e-5); the script
           exits with status 3 after printing if they are exceeded;
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
           workload (about 10 s: whole heads, or the sampled rows of the
           long-context workload, with rows/s and a labelled extrapolation
           to every row), on this host's cores.

Other flags: --no-cpu-baseline, --no-gemm-ceiling (skip the library bf16 GEMM
that measures the sustained matrix-core rate next to the published peak),
--copy-calibration (a plain device copy of known size, run under rocprofv3
--pmc to calibrate the byte counters), --pass bwd (time the backward instead:
one step = one attn_bwd / attn_bwd_blocksparse call on the workload's shapes,
10*d flops per allowed pair for the recomputed S and the dP, dV, dK, dQ
products; its cpu_baseline is the float64 gradient oracle), --pass select
(one step = the device mean-pooled selector, --topk blocks of 128 per query
block, then the block-sparse forward on its output, on the workload's shapes
with causal masking; reports the selector's cost against the dense tiles it
lets the forward skip), --pass splitkv (one step = attn_fwd_splitkv over --splits
key ranges in one launch, then the merge of the fp32 partial states).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded input recipes: shapes, seeds, block lists)

PEAK_BF16_TFLOPS = 2516.6    # 256 CU x 4096 bf16 FLOP/clk/CU x 2.4 GHz, dense
PEAK_F32_MFMA_TFLOPS = 157.3  # MI355X fp32 matrix peak, dense
# The softmax's vector work per executed score in the bf16 kernel: one FMA (scale
# and reference value), one v_exp_f32 (two issue slots on gfx950), one add to
# the fp32 denominator and half a bf16 pack: 4.5 wave64 instructions of 4 cycles
# per 64 scores on a 16-lane SIMD.
VALU_CYCLES_PER_SCORE = 4.5 * 4 / 64
# Issue cycles a 32x32x16 bf16 MFMA takes from its wave's instruction stream
# (a register-only probe, one wave per SIMD: 16 MFMAs take 512 cycles alone, 576
# with 96 FMAs between them, 688 with 128, 940 with 192).  A 32 x 32 score block
# needs d / 8 of them (d / 16 for the scores, d / 16 for its share of P V).
MFMA_ISSUE_CYCLES = 11
# Timed steps whose launch is bracketed by a HIP event pair (the first and then
# every EVENT_STRIDE-th): enough samples for the kernel's mean duration, few
# enough event records that they hardly add to the steps' wall clock.
EVENT_STRIDE = 8
SIMDS, CLOCK_GHZ = 256 * 4, 2.4
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}   # max|dO|, max|dLSE| against the oracle
CHECK_ROWS = 64              # seeded query rows per head the bench output is checked on
# the forward kernel's source and the headers it includes: the recorded counters stay valid
# only while none of them changes
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_softmax_attn_amd", "csrc", f)
                  for f in ("fwd_bf16.hip", "fwd_bf16_w64.hip", "fwd_common.h", "gfx950_util.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "{kernel}_{workload}_traffic.json")


def fwd_kernel_name(cfg) -> str:
    """The forward kernel the library launches for a workload (its dispatch
    rule: bf16 dense and causal d = 128 launches of at least 1024 256-row
    query tiles with N a multiple of 64 use the 64-row kernel unless
    ATTN_W64=0)."""
    if cfg.dtype != "bf16":
        return "fwd_f32_kernel"
    large = (cfg.N + 255) // 256 * cfg.B * cfg.H >= 1024 or os.environ.get("ATTN_TILE") == "256"
    if (not cfg.sparse and cfg.d == 128 and cfg.N >= 128 and cfg.N % 64 == 0 and large
            and os.environ.get("ATTN_TILE") != "128" and os.environ.get("ATTN_W64") != "0"):
        return "fwd_w64_kernel"
    return "fwd_bf16_kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def allowed_pairs_dense(cfg) -> int:
    per_head = cfg.N * (cfg.N + 1) // 2 if cfg.causal else cfg.N * cfg.N
    return cfg.B * cfg.H * per_head


def read_traffic(workload: str, kernel: str = "fwd_bf16"):
    path = TRAFFIC_FILE.format(workload=workload, kernel=kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None   # counters were taken on another version of the kernel
    return rec.get("traffic_bytes_per_launch")


def host_cores() -> dict:
    """The host cores this process may run on, and the BLAS threads numpy uses."""
    from threadpoolctl import threadpool_info
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"cores": len(os.sched_getaffinity(0)),
            "blas_threads": int(max([p.get("num_threads", 1) for p in blas] or [1])),
            "blas": ",".join(sorted({str(p.get("internal_api", "?")) for p in blas})) or "none"}


def cpu_baseline(cfg, q, k, v, budget_s: float = 10.0):
    """The oracle as it stands on a bounded sample of the same inputs: whole
    heads until the time budget is spent (at least one head), or, for the
    workloads checked on sampled rows, the sampled rows of each head."""
    import numpy as np
    import oracle

    hc = host_cores()
    done_heads, flops, rows_done, t_total = 0, 0, 0, 0.0
    H = cfg.H
    for h in range(H):
        qh, kh, vh = (t[:, h:h + 1].to("cpu") for t in (q, k, v))
        rows = workloads.config_rows(cfg, h)
        t0 = time.perf_counter()
        oracle.attn_fwd(qh, kh, vh, cfg.scale, cfg.causal, rows=rows)
        t_total += time.perf_counter() - t0
        done_heads += 1
        r = np.arange(cfg.N) if rows is None else np.asarray(rows)
        rows_done += len(r) * cfg.B
        pairs = int(np.sum(r + 1)) if cfg.causal else len(r) * cfg.N
        flops += 4 * cfg.d * pairs * cfg.B
        if t_total >= budget_s:
            break
    rec = {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": hc["cores"],
        "blas_threads": hc["blas_threads"],
        "kind": "oracle",
        "rows_per_s": round(rows_done / t_total, 1),
    }
    if cfg.sample_rows:
        total_rows = cfg.B * cfg.H * cfg.N
        rec["sample"] = (f"{cfg.sample_rows} sampled query rows of each of {done_heads} of {cfg.B * H} (batch, head) "
                         f"pairs of {cfg.name} (every key of each row), float64 numpy three-stage oracle, "
                         f"{t_total:.1f} s")
        rec["extrapolated_all_rows_s"] = round(total_rows / (rows_done / t_total), 1)
        rec["extrapolation"] = ("every row of every head at this row rate; rows later in a causal sequence "
                                "have more keys, so this understates the full cost")
    else:
        rec["sample"] = (f"{done_heads} of {cfg.B * H} (batch, head) pairs of {cfg.name}, every query row, "
                         f"float64 numpy three-stage oracle, {t_total:.1f} s")
    return rec


def oracle_check(cfg, q, k, v, o, lse, rows_per_head: int = CHECK_ROWS, mask_lists=None):
    """max|dO| and max|dLSE| of a forward's output against the float64 oracle
    on seeded query rows of every head (empty rows must be exactly O = 0 and
    LSE = -inf; any NaN fails)."""
    import numpy as np
    import oracle

    tol_o, tol_l = TOL[cfg.dtype]
    worst_o = worst_l = 0.0
    ok = True
    for b in range(cfg.B):
        for h in range(cfg.H):
            rows = workloads.sample_rows(cfg.N, min(rows_per_head, cfg.N), 77 * 1000 + b * cfg.H + h)
            qh, kh, vh = (t[b:b + 1, h:h + 1].to("cpu") for t in (q, k, v))
            if mask_lists is None:
                ro, rl = oracle.attn_fwd(qh, kh, vh, cfg.scale, cfg.causal, rows=rows)
            else:
                rp, col = mask_lists
                ro, rl = oracle.attn_fwd_blocksparse(qh, kh, vh, cfg.scale, cfg.causal, cfg.block, rp, col, 1,
                                                     rows=rows)
            ro, rl = ro[0], rl[0]
            go = o[b, h, rows].double().cpu().numpy()
            gl = lse[b, h, rows].double().cpu().numpy()
            live = np.isfinite(rl)
            if np.isnan(go).any() or np.isnan(gl).any():
                ok = False
            if not np.array_equal(np.isfinite(gl), live) or not np.all(go[~live] == 0) \
                    or not np.all(gl[~live] == -np.inf):
                ok = False
            if live.any():
                worst_o = max(worst_o, float(np.abs(go[live] - ro[live]).max()))
                worst_l = max(worst_l, float(np.abs(gl[live] - rl[live]).max()))
    ok = ok and worst_o <= tol_o and worst_l <= tol_l
    return {"rows_per_head": min(rows_per_head, cfg.N), "max_abs_dO": worst_o, "max_abs_dLSE": worst_l,
            "tol_O": tol_o, "tol_LSE": tol_l, "ok": bool(ok), "reference": "float64 oracle, seeded rows"}


def gemm_ceiling(n: int = 8192, reps: int = 20):
    """Sustained bf16 matrix-core rate of this GPU on random operands, from a
    plain library GEMM (torch.matmul, n x n x n): context for the roofline,
    since the published peak assumes a clock the chip does not hold under a
    sustained bf16 matrix load."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    return {"what": f"torch.matmul bf16 {n}x{n}x{n}, random N(0,1) operands", "tflops": round(2 * n ** 3 / ms / 1e9, 1)}


def copy_calibration(nbytes: int = 1 << 30):
    """A plain device-to-device copy of known size (torch's copy kernel)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "dispatches": 3}))


def algorithmic_bytes(cfg, mask=None) -> int:
    """Bytes the method itself must move per launch: Q read once, O written
    once, 4 B of LSE per row, and K and V read once -- for a block-sparse
    pattern only the key blocks its lists reference (one pattern for every
    head here)."""
    elem = 2 if cfg.dtype == "bf16" else 4
    rows = cfg.B * cfg.H * cfg.N
    qo = 2 * rows * cfg.d * elem + 4 * rows
    if mask is None:
        return qo + 2 * rows * cfg.d * elem
    keys = 0
    for kb in sorted(set(int(c) for c in mask.col)):
        keys += min(cfg.N, (kb + 1) * cfg.block) - kb * cfg.block
    return qo + 2 * cfg.B * cfg.H * keys * cfg.d * elem


def device_info(dev):
    """The GPU's compute-unit count and maximum clock (rocminfo, when it runs;
    the CU count also from the runtime), and the bf16 matrix peak they give."""
    import subprocess
    import torch
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus_runtime": props.multi_processor_count, "cus_rocminfo": None, "max_clock_mhz_rocminfo": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        for agent in out.split("*******")[1:]:
            fields = {}
            for line in agent.splitlines():
                if ":" in line:
                    key, _, val = line.partition(":")
                    fields.setdefault(key.strip(), val.strip())
            if fields.get("Name", "").startswith("gfx"):
                info["cus_rocminfo"] = int(fields["Compute Unit"])
                info["max_clock_mhz_rocminfo"] = int(fields["Max Clock Freq. (MHz)"])
                break
    except (OSError, subprocess.SubprocessError, KeyError, ValueError):
        pass
    cus = info["cus_rocminfo"] or info["cus_runtime"]
    if cus and info["max_clock_mhz_rocminfo"]:
        info["bf16_peak_tflops_from_units"] = round(cus * 4096 * info["max_clock_mhz_rocminfo"] * 1e6 / 1e12, 1)
    return info


def vector_floor(executed_scores: int, mean_launch_ms: float, d: int = 0) -> dict:
    """Time floors of a launch at 2.4 GHz on all 1024 SIMDs: the softmax's
    vector work (VALU_CYCLES_PER_SCORE per executed score), and with the head
    dimension d the issue floor of one wave's instruction stream (that vector
    work plus MFMA_ISSUE_CYCLES for each of the d / 8 MFMAs of a 32 x 32 score
    block); the launch's time against each.  The matrix work's floor (4 d flops
    per score at the bf16 peak) is added by the caller."""
    unit = SIMDS * CLOCK_GHZ * 1e9
    floor_ms = executed_scores * VALU_CYCLES_PER_SCORE / unit * 1e3
    rec = {"cycles_per_score": VALU_CYCLES_PER_SCORE, "floor_ms": round(floor_ms, 5),
           "frac": round(floor_ms / mean_launch_ms, 4)}
    if d:
        issue = VALU_CYCLES_PER_SCORE + MFMA_ISSUE_CYCLES * (d / 8) / 1024
        issue_ms = executed_scores * issue / unit * 1e3
        rec.update({"issue_cycles_per_score": round(issue, 5), "issue_floor_ms": round(issue_ms, 5),
                    "issue_frac": round(issue_ms / mean_launch_ms, 4)})
    return rec


def executed_tiles_128(cfg, mask=None) -> int:
    """Executed work of a causal or block-sparse run in b x b tiles (b = 128;
    the sparse pattern's own block): diagonal tiles count whole."""
    if mask is not None:
        return int(mask.executed_tile_pairs[0]) * cfg.B * cfg.H
    nb = -(-cfg.N // 128)
    return cfg.B * cfg.H * nb * (nb + 1) // 2


def bench_fwd(args, cfg, dev, gemm=None):
    """One workload's record: timed steps of the one-call forward, then the
    oracle check of the timed output, then the CPU baseline."""
    import torch
    import block_sparse_softmax_attn_amd as attn

    tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    q, k, v = (torch.randn((cfg.B, cfg.H, cfg.N, cfg.d), generator=gen, device=dev, dtype=torch.float32)
               .to(tdtype).contiguous() for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), device=dev, dtype=torch.float32)

    # One step = one call of the one-call entry point: a single launch of the
    # fused kernel, timed with HIP events on the launch stream.
    mask_lists = None
    if cfg.sparse:
        rp, col = workloads.config_block_lists(cfg)
        mask_lists = (rp, col)
        t0 = time.perf_counter()
        mask = attn.blockmask_build(rp, col, 1, cfg.N, cfg.block, cfg.causal)
        build_ms = (time.perf_counter() - t0) * 1e3
        pairs = int(mask.allowed_pairs[0]) * cfg.B * cfg.H
        executed = executed_tiles_128(cfg, mask) * cfg.block * cfg.block
        alg_bytes = algorithmic_bytes(cfg, mask)
        mask.to_device(dev)
        fused = lambda: attn.attn_fwd_blocksparse(q, k, v, mask, scale=cfg.scale, causal=cfg.causal,
                                                  out=o, lse=lse)
    else:
        build_ms = None
        pairs = allowed_pairs_dense(cfg)
        executed = executed_tiles_128(cfg) * 128 * 128 if cfg.causal else None
        alg_bytes = algorithmic_bytes(cfg)
        fused = lambda: attn.attn_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, out=o, lse=lse)
    flops = 4 * cfg.d * pairs

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(0, args.steps, EVENT_STRIDE)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % EVENT_STRIDE == 0:
            ev[i // EVENT_STRIDE][0].record(stream)
            fused()
            ev[i // EVENT_STRIDE][1].record(stream)
        else:
            fused()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch = sorted(e[0].elapsed_time(e[1]) for e in ev)
    mean_launch_ms = sum(launch) / len(launch)
    median_launch_ms = launch[len(launch) // 2] if len(launch) % 2 else 0.5 * (launch[len(launch) // 2 - 1] +
                                                                              launch[len(launch) // 2])
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    value = flops * args.steps / wall / 1e12
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s (allowed pairs) + % of bf16 MFMA peak, 1\u00d7MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": cfg.description,
            "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "causal": cfg.causal,
            "block_sparse": cfg.sparse, "scale": cfg.scale, "seed": cfg.seed,
            "allowed_pairs": pairs, "flops_per_step": flops,
            "flop_count": "4*d per allowed (query, key) pair",
            "parallelism": "single GPU",
        },
        "timing": {"launch_ms_mean": round(mean_launch_ms, 5), "launch_ms_median": round(median_launch_ms, 5),
                   "launch_ms_min": round(launch[0], 5), "launches": len(launch),
                   "launches_timed_of": args.steps, "event_stride": EVENT_STRIDE},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": (read_traffic(cfg.name, fwd_kernel_name(cfg).replace("_kernel", "")) if cfg.dtype == "bf16"
                        else None),
            "kernel": fwd_kernel_name(cfg),
            "mean_launch_ms": round(mean_launch_ms, 5),
            # HBM rates per launch: the method's own bytes, and the counted bytes when known
            "algorithmic_bytes": alg_bytes,
            "hbm_gbps_algorithmic": round(alg_bytes / (mean_launch_ms * 1e-3) / 1e9, 1),
        },
    }
    if rec["roofline"]["traffic"] is not None:
        rec["roofline"]["hbm_gbps_counted"] = round(rec["roofline"]["traffic"] / (mean_launch_ms * 1e-3) / 1e9, 1)
    if cfg.dtype == "bf16":
        # secondary bound: the softmax's vector work on the executed scores
        # (whole tiles for causal and block-sparse runs); at d = 64 it exceeds
        # the matrix work's time at peak
        scores = executed if executed is not None else pairs
        vf = vector_floor(scores, mean_launch_ms, cfg.d)
        vf["mfma_floor_ms"] = round(4 * cfg.d * scores / (PEAK_BF16_TFLOPS * 1e12) * 1e3, 5)
        vf["binding"] = "valu" if vf["floor_ms"] > vf["mfma_floor_ms"] else "mfma"
        vf["binding_with_issue"] = "issue" if vf["issue_floor_ms"] > vf["mfma_floor_ms"] else "mfma"
        rec["roofline"]["vector_floor"] = vf
    if cfg.dtype != "bf16":
        rec["roofline"]["note"] = ("fp32 workload of 16.8 MFLOP: one small launch, latency-bound; "
                                   "its time is reported for context, against the fp32 matrix peak")
    if executed is not None:
        rec["config"]["executed_tile_pairs_128"] = executed // (cfg.block * cfg.block if cfg.sparse else 128 * 128)
        rec["config"]["executed_tile_flops_per_step"] = 4 * cfg.d * executed
        rec["config"]["executed_tile_tflops"] = round(4 * cfg.d * executed * args.steps / wall / 1e12, 3)
    if build_ms is not None:
        rec["config"]["blockmask_build_ms_host"] = round(build_ms, 3)
    if gemm is not None:
        rec["roofline"]["measured_bf16_gemm_ceiling"] = gemm
    rec["check"] = oracle_check(cfg, q, k, v, o, lse, mask_lists=mask_lists)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, q, k, v)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense-h32-n8192-d128", choices=list(workloads.CONFIGS))
    ap.add_argument("--all", action="store_true", help="one line per workload (every config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-ceiling", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd", "select", "splitkv"])
    ap.add_argument("--topk", type=int, default=16)
    ap.add_argument("--splits", type=int, default=8)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the attention forward is measured on one MI355X; sharding is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import block_sparse_softmax_attn_amd as attn  # noqa: F401  (fails loudly without the built library)

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    cfg = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.which != "fwd" and cfg.dtype != "bf16":
        print(f"--pass {args.which} takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    if args.which == "bwd":
        bench_bwd(args, cfg, dev)
        return
    if args.which == "splitkv":
        bench_splitkv(args, cfg, dev)
        return
    if args.which == "select":
        bench_select(args, cfg, dev)
        return
    gemm = None if args.no_gemm_ceiling else gemm_ceiling()
    device = device_info(dev)
    failed = False
    for c in (workloads.CONFIGS.values() if args.all else [cfg]):
        rec = bench_fwd(args, c, dev, gemm)
        rec["device"] = device
        failed = failed or not rec["check"]["ok"]
        print(json.dumps(rec), flush=True)
    if failed:
        print("bench.py: the timed output exceeds the oracle tolerance (see \"check\")", file=sys.stderr)
        sys.exit(3)


def cpu_baseline_bwd(cfg, q, k, v, do, mask_lists, budget_s: float = 10.0):
    """The gradient oracle as it stands, on whole heads, until the budget is spent."""
    import oracle
    hc = host_cores()
    done, flops, t_total = 0, 0, 0.0
    for h in range(cfg.H):
        qh, kh, vh, dh = (t[:, h:h + 1].to("cpu") for t in (q, k, v, do))
        t0 = time.perf_counter()
        if mask_lists is None:
            oracle.attn_bwd(qh, kh, vh, dh, cfg.scale, cfg.causal)
        else:
            rp, col, pairs_head = mask_lists
            oracle.attn_bwd_blocksparse(qh, kh, vh, dh, cfg.scale, cfg.causal, cfg.block, rp, col, 1)
        t_total += time.perf_counter() - t0
        done += 1
        per_head = (mask_lists[2] if mask_lists is not None
                    else (cfg.N * (cfg.N + 1) // 2 if cfg.causal else cfg.N * cfg.N))
        flops += 10 * cfg.d * per_head * cfg.B
        if t_total >= budget_s:
            break
    return {
        "value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": hc["cores"],
        "blas_threads": hc["blas_threads"], "kind": "oracle",
        "sample": f"{done} of {cfg.B * cfg.H} (batch, head) pairs of {cfg.name}, float64 numpy gradient oracle "
                  f"(forward recomputed), {t_total:.1f} s",
    }


def bench_bwd(args, cfg, dev):
    """One step = one backward call on inputs resident in HBM (forward outputs
    computed once, untimed)."""
    import torch
    import block_sparse_softmax_attn_amd as attn

    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    q, k, v, do = (torch.randn((cfg.B, cfg.H, cfg.N, cfg.d), generator=gen, device=dev, dtype=torch.float32)
                   .to(torch.bfloat16).contiguous() for _ in range(4))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    if cfg.sparse:
        rp, col = workloads.config_block_lists(cfg)
        mask = attn.blockmask_build(rp, col, 1, cfg.N, cfg.block, cfg.causal)
        ws = torch.empty(attn.bwd_blocksparse_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, mask), dtype=torch.uint8,
                         device=dev)
        pairs_head = int(mask.allowed_pairs[0])
        o, lse = attn.attn_fwd_blocksparse(q, k, v, mask, scale=cfg.scale, causal=cfg.causal)
        step = lambda: attn.attn_bwd_blocksparse(q, k, v, o, lse, do, mask, scale=cfg.scale, causal=cfg.causal,
                                                 dq=dq, dk=dk, dv=dv, workspace=ws)
        mask_lists = (rp, col, pairs_head)
    else:
        ws = torch.empty(attn.bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.uint8, device=dev)
        pairs_head = cfg.N * (cfg.N + 1) // 2 if cfg.causal else cfg.N * cfg.N
        o, lse = attn.attn_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal)
        step = lambda: attn.attn_bwd(q, k, v, o, lse, do, scale=cfg.scale, causal=cfg.causal,
                                     dq=dq, dk=dk, dv=dv, workspace=ws)
        mask_lists = None
    pairs = pairs_head * cfg.B * cfg.H
    flops = 10 * cfg.d * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    value = flops * args.steps / wall / 1e12
    achieved = flops / (mean_ms * 1e-3) / 1e12
    rec = {
        "metric": "attention bwd TFLOP/s (allowed pairs, 10*d flops per pair) + % of bf16 MFMA peak, 1\u00d7MI355X",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": cfg.description, "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
                   "causal": cfg.causal, "block_sparse": cfg.sparse, "scale": cfg.scale, "seed": cfg.seed,
                   "allowed_pairs": pairs, "flops_per_step": flops,
                   "flop_count": "10*d per allowed (query, key) pair: S recomputed, dP, dV, dK, dQ",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_bwd call: row statistics, dK/dV kernel, dQ kernel",
                     "mean_call_ms": round(mean_ms, 5)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_bwd(cfg, q, k, v, do, mask_lists)
    print(json.dumps(rec), flush=True)


def _time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3, sum(e[0].elapsed_time(e[1]) for e in ev) / steps


def bench_select(args, cfg, dev):
    """Selector + block-sparse forward against the dense causal forward on the
    workload's shapes (block 128)."""
    import torch
    import block_sparse_softmax_attn_amd as attn

    block, topk = 128, int(args.topk)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    q, k, v = (torch.randn((cfg.B, cfg.H, cfg.N, cfg.d), generator=gen, device=dev, dtype=torch.float32)
               .to(torch.bfloat16).contiguous() for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    lib = attn._get_lib()
    sel_ws = torch.empty(lib.attn_select_meanpool_workspace_bytes(cfg.B, cfg.H, cfg.H, cfg.N, cfg.d, block),
                         dtype=torch.uint8, device=dev)
    state = {}

    def select():
        state["mask"] = attn.select_meanpool(q, k, block, topk, causal=True, scale=cfg.scale, workspace=sel_ws)

    def step():
        select()
        attn.attn_fwd_blocksparse(q, k, v, state["mask"], scale=cfg.scale, causal=True, out=o, lse=lse)

    select()
    mask = state["mask"]
    pairs = int(mask.allowed_pairs.sum())       # one count per (batch, head) pattern
    executed_tiles = int(mask.executed_tile_pairs.sum())
    nb = -(-cfg.N // block)
    dense_tiles = cfg.B * cfg.H * nb * (nb + 1) // 2
    wall_ms, step_ms = _time_calls(step, args.steps, args.warmup, stream)
    _, sel_ms = _time_calls(select, args.steps, args.warmup, stream)
    _, dense_ms = _time_calls(lambda: attn.attn_fwd(q, k, v, scale=cfg.scale, causal=True, out=o, lse=lse),
                              max(3, args.steps // 10), 2, stream)
    flops = 4 * cfg.d * pairs
    skipped = dense_tiles - executed_tiles
    rec = {
        "metric": "attention fwd TFLOP/s (allowed pairs of the selected pattern, selector included), 1\u00d7MI355X",
        "value": round(flops / (wall_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.description + f", mean-pooled top-{topk} of 128-token blocks, causal",
                   "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "block": block, "topk": topk,
                   "allowed_pairs": pairs, "executed_tiles": executed_tiles, "dense_causal_tiles": dense_tiles,
                   "parallelism": "single GPU"},
        "selector": {"mean_ms": round(sel_ms, 5), "dense_causal_forward_ms": round(dense_ms, 4),
                     "skipped_tiles": skipped,
                     "skipped_tile_time_ms_estimate": round(dense_ms * skipped / dense_tiles, 4),
                     "selector_cost_over_skipped_work": round(sel_ms / (dense_ms * skipped / dense_tiles), 5),
                     "step_speedup_over_dense": round(dense_ms / step_ms, 3)},
    }
    print(json.dumps(rec), flush=True)


def bench_splitkv(args, cfg, dev):
    """One step = attn_fwd_splitkv: the forward over --splits key ranges in one
    launch (fp32 partial states in the workspace), then the merge launch."""
    import torch
    import block_sparse_softmax_attn_amd as attn

    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    q, k, v = (torch.randn((cfg.B, cfg.H, cfg.N, cfg.d), generator=gen, device=dev, dtype=torch.float32)
               .to(torch.bfloat16).contiguous() for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), device=dev, dtype=torch.float32)
    lib = attn._get_lib()
    ws = torch.empty(lib.attn_fwd_splitkv_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, 1, args.splits),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    step = lambda: attn.attn_fwd_splitkv(q, k, v, scale=cfg.scale, causal=cfg.causal, num_splits=args.splits,
                                         out=o, lse=lse, workspace=ws)
    wall_ms, _ = _time_calls(step, args.steps, args.warmup, stream)
    pairs = allowed_pairs_dense(cfg)
    rows = cfg.B * cfg.H * cfg.N
    merge_bytes = args.splits * rows * (cfg.d * 4 + 4) + rows * (cfg.d * 2 + 4)
    rec = {
        "metric": "attention fwd TFLOP/s (allowed pairs), key ranges in one launch + merge, 1\u00d7MI355X",
        "value": round(4 * cfg.d * pairs / (wall_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.description + f", {args.splits} key ranges", "B": cfg.B, "H": cfg.H,
                   "N": cfg.N, "d": cfg.d, "causal": cfg.causal, "splits": args.splits,
                   "merge_bytes_per_step": merge_bytes, "parallelism": "single GPU"},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
