"""Benchmark: BigBird block-sparse attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode cold|warm]
                    [--launch fused|split] [--no-cpu-baseline] [--copy-calibration]
    python bench.py --pass backward [--steps K] [--warmup W] [--workload NAME] [--mode cold|warm]
    python bench.py --pmc-summary FETCH_CSV WRITE_CSV --workload NAME --command "..."

`--pass layer` times bb_layer_forward: the QKV projection, the attention and
the output projection of the layer (hidden = H*64, synthetic weights); its
useful FLOPs add 2*M*N*K per projection (M = B*L) to the attention's.
`--pass stack` times bb_layer_stack_forward over --layers layers (default 12,
BigBird-base's depth), layer l with its own weights and the random table
seeded with l; the layers feed each other, so the call is timed warm.

`--query-mask` runs the forward (or, with `--pass backward`, the forward
with the log-sum-exp and the backward) with BB_QUERY_MASK (the query-side
padding variant: a pair is masked when its query or its key is padding).

`--pass backward` times bb_attn_backward instead (the default is the forward,
the headline): one step = one backward call over the whole batch (the dQ
pass, which also forms D and LSE2, the dK/dV pass, the split-K reduce), its inputs (q, k, v,
out, dout, lse from one forward) resident in HBM.  Useful backward FLOPs are
10*d per attended pair -- the five products of the recompute-based backward
(S, dP, dV, dK, dQ); the kernels execute 14*d (S and dP in both passes).

One step = one bb_attn_forward call over the whole batch: key pad bias, tile
lists, HBM->LDS staging, QK^T, online softmax, PV, the split-K global rows and
their merge -- every per-call step of the hot path.  The random-block table is
built once on the host beforehand, as the reference builds it once at layer
construction; its build time is reported separately.

Before the W warm-up calls, a W below CLOCK_SETTLE's count gets untimed
calls up to that count (about 30 ms of kernels), so that the timed region
starts at full engine clock; their number is config.clock_settle_calls.

Prints ONE JSON line.  `value` is useful TFLOP/s: 4*d FLOPs per attended
(query, key) pair, pairs counted from the block pattern (padding included),
over the wall time of K timed steps (hipEvents on the launch stream, device
synchronised on both sides, inputs already resident in HBM).  Cold mode
rotates among input sets whose total footprint exceeds twice the 256 MB
last-level cache, so each call reads HBM.

`roofline` is for the dominant kernel (the fused work-unit kernel, which does
every useful FLOP): a second pass runs the same K steps through the two-phase
form of the call, each kernel timestamped at its start and end by its own
launch (hipExtLaunchKernel events on the launch stream), so the kernel's
execution time is measured without enqueue gaps (mean, and p10 / median /
p90 over the K launches).  `traffic` is the HBM bytes per launch from
the committed rocprofv3 counter summary, used only if that summary was taken
on the current kernel source.  `cpu_baseline` times the fp64 oracle on a
bounded sample of (batch, head) units of the same workload on this host.
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
sys.path.insert(0, ROOT)

METRIC = "useful TFLOP/s + tokens/s, BigBird attn fwd L=4096 H=12 d=64 bf16, 1 GPU"
DEFAULT_WORKLOAD = "base_B4_H12_L4096_pad"   # the workload METRIC is quoted on
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBPS = 8000.0
LLC_BYTES = 256 * 2**20
COPY_BYTES = 512 * 2**20                        # copy-kernel calibration size
MFMA_CALIB_N = 8192                             # bf16 GEMM calibration: 2 n^3 FLOPs
KERNEL_SRC = os.path.join(ROOT, "block_sparse_long_bigbird_amd", "csrc", "bb_attn.hip")
BUILD_SCRIPT = os.path.join(ROOT, "block_sparse_long_bigbird_amd", "build.py")
PROFILES = os.path.join(ROOT, "profiles")
MAIN_KERNEL = "bb_fused_kernel"
# Untimed calls made before the W warm-up calls when W is smaller (about 30 ms
# of kernels per pass): the engine clock ramps up over the first milliseconds
# of load, and a timed region that starts below full clock reads low (10
# warm-up calls: 431 useful TFLOP/s on the headline shape; 500: 521).  The
# count is reported as config.clock_settle_calls; the timed region is always
# exactly K calls.
CLOCK_SETTLE = {"forward": 500, "backward": 200, "layer": 200, "stack": 20}


def settle_calls(args, which: str) -> int:
    return max(0, CLOCK_SETTLE[which] - args.warmup)


def pairs_per_unit(L: int, block: int, r: int):
    """Attended (query, key) pairs of one (batch, head): (global rows, middle rows)."""
    nb = L // block
    glob = 2 * block * L
    mid = block * block * ((nb - 4) * (5 + r) + 2 * (4 + r))
    return glob, mid


def useful_flops(w):
    g, m = pairs_per_unit(w.L, w.block, w.r)
    return 4 * w.d * (g + m) * w.B * w.H


def algorithmic_bytes(w):
    es = 2 if w.dtype == "bf16" else 4
    b = 4 * w.B * w.H * w.L * w.d * es
    if w.pad != "none":
        b += w.B * w.L
    b += 4 * w.H * (w.nb - 2) * w.r
    return b


# The forward kernels and every device helper they use come first in the
# source; the backward and layer sections follow this marker and do not change
# the forward's code.
FORWARD_END = b"// ================================================================ backward =="


def source_sha256() -> str:
    """sha256 of the forward part of the kernel source (up to FORWARD_END)
    followed by the build script (its compiler flags shape the same kernel)."""
    with open(KERNEL_SRC, "rb") as f:
        text = f.read()
    cut = text.find(FORWARD_END)
    with open(BUILD_SCRIPT, "rb") as f:
        build = f.read()
    return hashlib.sha256((text if cut < 0 else text[:cut]) + build).hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{MAIN_KERNEL}_{workload}.txt")


def committed_traffic(workload: str):
    """HBM bytes per launch from profiles/, if measured on the current kernel source."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, command: str) -> None:
    """Turn two rocprofv3 --pmc counter CSVs into the committed traffic summary.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the main kernel are each
    scaled by the factor that makes the same counter read exactly COPY_BYTES
    for the calibration copy kernel that bench.py --copy-calibration runs.
    """
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    def pick(vals, key):
        names = [n for n in vals if key in n]
        if not names:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}")
        return statistics.mean(v for n in names for v in vals[n]), sum(len(vals[n]) for n in names)

    from block_sparse_long_bigbird_amd.workloads import WORKLOADS
    w = WORKLOADS[workload]
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    # The calibration copy moves COPY_BYTES in and COPY_BYTES out.  Other copy
    # dispatches (input-set clones) are far smaller, so keep the copy-kernel
    # dispatches within 25% of the largest one.
    def calib(vals):
        keys = [n for n in vals if "copy" in n.lower()]
        if not keys:
            raise SystemExit("no copy-kernel dispatch found (run bench.py with --copy-calibration)")
        allv = [(x, n) for n in keys for x in vals[n]]
        top = max(x for x, _ in allv)
        big = [x for x, _ in allv if x >= 0.75 * top]
        name = max(allv)[1]
        return statistics.median(big) * 1024.0, name
    copy_fetch, copy_key = calib(f)
    copy_write, _ = calib(wr)
    kf, nf = pick(f, MAIN_KERNEL)
    kw, nw = pick(wr, MAIN_KERNEL)
    ffac, wfac = COPY_BYTES / copy_fetch, COPY_BYTES / copy_write
    fetch_b, write_b = kf * 1024.0 * ffac, kw * 1024.0 * wfac
    lines = [
        f"# HBM traffic of {MAIN_KERNEL} on {workload} (rocprofv3 --pmc, one counter per run)",
        f"command: {command}",
        f"source_sha256: {source_sha256()}",
        f"dispatches: FETCH_SIZE {nf}, WRITE_SIZE {nw}",
        f"fetch_kib_per_dispatch: {kf:.1f}",
        f"write_kib_per_dispatch: {kw:.1f}",
        f"copy_kernel: {copy_key[:80]}",
        f"copy_bytes: {COPY_BYTES}",
        f"copy_fetch_kib: {copy_fetch / 1024.0:.1f}",
        f"copy_write_kib: {copy_write / 1024.0:.1f}",
        f"fetch_scale: {ffac:.4f}",
        f"write_scale: {wfac:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_call: {algorithmic_bytes(w)}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / algorithmic_bytes(w):.3f}",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _oracle_waves(w, run_units, budget_s: float):
    """Run the oracle on (b, h) units in waves of one unit per worker thread
    until `budget_s` is spent (at least one wave).  Returns (units done, seconds,
    workers)."""
    from oracle.parallel import host_workers
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    n = host_workers()
    done = 0
    t0 = time.perf_counter()
    while done < len(units):
        run_units(units[done:done + n], n)
        done = min(len(units), done + n)
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0, n


def _baseline_fields(w, done, el, n, flops_per_job, what):
    frac = done / (w.B * w.H)
    return {
        "value": round(flops_per_job * frac / el / 1e12, 6),
        "unit": "TFLOP/s",
        "tokens_per_s": round(w.tokens * frac / el, 1),
        "cores": int(n),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) units of {w.name}, {what} of all {w.L} query rows "
                  f"each, fp64 numpy, {el:.1f} s",
        "parallelism": f"{n} worker threads over (batch, head) units, BLAS 1 thread each",
        "host_cpus_visible": len(os.sched_getaffinity(0)),
    }


def mfma_path(workload: str) -> str:
    return os.path.join(PROFILES, f"mfma_counters_{MAIN_KERNEL}_{workload}.txt")


def pmc_mfma_summary(csv_path: str, workload: str, command: str) -> None:
    """Turn one rocprofv3 --pmc CSV (MFMA, VALU, SALU and clock counters of a
    bench run with --mfma-calibration) into the committed MFMA summary.

    SQ_INSTS_VALU_MFMA_MOPS_BF16 is converted to FLOPs with the factor that
    makes it read exactly 2 n^3 for the calibration GEMM (torch.matmul, n =
    MFMA_CALIB_N); the kernel's duration is End - Start of each dispatch;
    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so GUI_ACTIVE / 8 / duration is
    the engine clock during the kernel and SQ_VALU_MFMA_BUSY_CYCLES over
    (SIMDs x GUI_ACTIVE / 8) the fraction of SIMD cycles the MFMA pipe is busy.
    """
    import csv
    import statistics

    from block_sparse_long_bigbird_amd.workloads import WORKLOADS
    w = WORKLOADS[workload]
    disp = {}
    for row in csv.DictReader(open(csv_path)):
        key = (row["Dispatch_Id"], row["Kernel_Name"])
        d = disp.setdefault(key, {"dur_ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
        d[row["Counter_Name"]] = float(row["Counter_Value"])

    def select(match):
        return [d for (_, name), d in disp.items() if match(name)]

    gemm = select(lambda n: n.startswith("Cijk") or "gemm" in n.lower())
    kern = select(lambda n: MAIN_KERNEL in n)
    if not gemm or not kern:
        raise SystemExit("need dispatches of the calibration GEMM and of the main kernel")
    n = MFMA_CALIB_N
    flop_per_mop = statistics.median(2.0 * n ** 3 / d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in gemm)
    simds = 256 * 4

    def stats(ds):
        dur = statistics.mean(d["dur_ns"] for d in ds)
        flops = statistics.mean(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds) * flop_per_mop
        gui = statistics.mean(d["GRBM_GUI_ACTIVE"] for d in ds) / 8
        busy = statistics.mean(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds)
        return dur, flops, gui, busy

    kd, kf, kg, kb = stats(kern)
    gd, gf, gg, gb = stats(gemm)
    useful = useful_flops(w)
    waves = statistics.mean(d.get("SQ_WAVES", 0.0) for d in kern)
    lines = [
        f"# MFMA counters of {MAIN_KERNEL} on {workload} (rocprofv3 --pmc, one run)",
        f"command: {command}",
        f"source_sha256: {source_sha256()}",
        f"dispatches: {len(kern)} of the kernel, {len(gemm)} of the calibration GEMM (bf16, n = {n})",
        f"flop_per_mops_bf16: {flop_per_mop:.3f}   (2 n^3 / SQ_INSTS_VALU_MFMA_MOPS_BF16 of the GEMM)",
        f"kernel_duration_us: {kd / 1e3:.3f}   (mean End - Start)",
        f"kernel_mfma_flop_per_launch: {kf:.6g}   (counter)",
        f"useful_flop_per_launch: {useful}   (algorithmic: 4 d per attended pair)",
        f"counter_over_useful: {kf / useful:.6f}",
        f"achieved_mfma_tflops: {kf / kd / 1e3:.1f}   (counter FLOPs / duration)",
        f"achieved_frac_of_peak: {kf / kd / 1e3 / PEAK_TFLOPS['bf16']:.4f}   (peak {PEAK_TFLOPS['bf16']} TFLOP/s at 2.4 GHz)",
        f"engine_clock_ghz: {kg / kd:.3f}   (GRBM_GUI_ACTIVE / 8 XCDs / duration)",
        f"mfma_busy_frac: {kb / (simds * kg):.4f}   (SQ_VALU_MFMA_BUSY_CYCLES / ({simds} SIMDs x cycles))",
        f"valu_insts_per_launch: {statistics.mean(d['SQ_INSTS_VALU'] for d in kern):.0f}",
        f"salu_insts_per_launch: {statistics.mean(d['SQ_INSTS_SALU'] for d in kern):.0f}",
        f"mfma_insts_per_launch: {statistics.mean(d['SQ_INSTS_MFMA'] for d in kern):.0f}",
        f"gemm_duration_us: {gd / 1e3:.1f}",
        f"gemm_achieved_tflops: {gf / gd / 1e3:.1f}",
        f"gemm_engine_clock_ghz: {gg / gd:.3f}",
        f"gemm_mfma_busy_frac: {gb / (simds * gg):.4f}",
    ]
    if waves:
        lines.append(f"waves_per_launch: {waves:.0f}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(mfma_path(workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(w, inputs, ri, budget_s: float, query_mask: bool = False):
    """Time the fp64 oracle on (b, h) units until `budget_s` is spent."""
    from oracle.parallel import forward_units
    q, k, v, pad = inputs
    qd, kd, vd = (t.float().numpy() for t in (q, k, v))
    pd = None if pad is None else pad.numpy()
    done, el, n = _oracle_waves(
        w, lambda units, n: forward_units(qd, kd, vd, pd, ri, w.block, units=units, workers=n,
                                          query_mask=query_mask), budget_s)
    return _baseline_fields(w, done, el, n, useful_flops(w), "forward")


def cpu_baseline_backward(w, inputs, dout, ri, budget_s: float, query_mask: bool = False):
    """Time the fp64 oracle's backward on (b, h) units until `budget_s` is spent."""
    from oracle.parallel import backward_units
    q, k, v, pad = inputs
    qd, kd, vd, gd = (t.float().numpy() for t in (q, k, v, dout))
    pd = None if pad is None else pad.numpy()
    done, el, n = _oracle_waves(
        w, lambda units, n: backward_units(qd, kd, vd, pd, ri, w.block, gd, units=units, workers=n,
                                           query_mask=query_mask),
        budget_s)
    return _baseline_fields(w, done, el, n, 2.5 * useful_flops(w), "backward")


def bench_layer(args, w, dev, stack=False):
    """One JSON line for bb_layer_forward, or with stack=True for
    bb_layer_stack_forward over args.layers layers (see the module docstring)."""
    import torch

    from block_sparse_long_bigbird_amd import binding as bb
    from block_sparse_long_bigbird_amd.workloads import make_layer_inputs, make_stack_weights

    hid = w.H * w.d
    x, w_qkv, b_qkv, w_o, b_o, pad = make_layer_inputs(w)
    dpad = None if pad is None else pad.to(dev)
    n_layers = args.layers if stack else 1
    if stack:
        tables = [bb.bb_rand_idx_build(l, w.H, w.L, w.block, w.r) for l in range(n_layers)]
        layers = [tuple(t.to(dev) for t in lw) + (torch.from_numpy(ri).to(dev) if w.r > 0 else None,)
                  for lw, ri in zip(make_stack_weights(w, n_layers), tables)]
        n = bb.bb_layer_stack_workspace_bytes(w.B, w.L, hid, w.H, w.block)
    else:
        ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
        dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
        weights = [t.to(dev) for t in (w_qkv, b_qkv, w_o, b_o)]
        n = bb.bb_layer_workspace_bytes(w.B, w.L, hid, w.H, w.block)
    x0 = x.to(dev)
    footprint = 2 * x0.numel() * x0.element_size()
    n_sets = 1 if args.mode == "warm" or stack else max(2, math.ceil(2.1 * LLC_BYTES / footprint))
    sets = [(x0 if i == 0 else x0.clone(), torch.empty_like(x0)) for i in range(n_sets)]
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call(i):
        xi, yi = sets[i % n_sets]
        if stack:
            bb.bb_layer_stack_forward(xi, layers, dpad, w.B, w.L, hid, w.H, w.block, w.r, yi, ws,
                                      stream=stream.cuda_stream)
        else:
            bb.bb_layer_forward(xi, *weights, dpad, dri, w.B, w.L, hid, w.H, w.block, w.r, yi, ws,
                                stream=stream.cuda_stream)

    settle = settle_calls(args, "stack" if stack else "layer")
    for i in range(settle + args.warmup):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    M = w.B * w.L
    proj = n_layers * (2 * M * (3 * hid) * hid + 2 * M * hid * hid)
    flops = n_layers * useful_flops(w) + proj
    value = flops / (ms * 1e-3) / 1e12
    what = (f"stack of {n_layers} attention layers, per-layer random tables" if stack
            else "attention layer")
    out = {
        "metric": f"useful TFLOP/s, BigBird {what} fwd (projections + attn) L={w.L} hidden={w.H * w.d} bf16, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "tokens_per_s": round(w.tokens / (ms * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/hidden) weights)",
        "config": {"workload": w.name, "pass": "stack" if stack else "layer", "layers": n_layers,
                   "B": w.B, "L": w.L, "hidden": hid, "H": w.H,
                   "block": w.block, "r": w.r, "pad": w.pad, "mode": "warm" if stack else args.mode,
                   "input_sets": n_sets, "clock_settle_calls": settle,
                   "useful_gflop_per_step": round(flops / 1e9, 4),
                   "projection_gflop_per_step": round(proj / 1e9, 4)},
        "roofline": {"bound": "mfma",
                     "kernel": f"whole {'stack' if stack else 'layer'} call (2 projections + attention per layer)",
                     "achieved": round(value, 3), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(value / PEAK_TFLOPS["bf16"], 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_backward(args, w, dev):
    """One JSON line for bb_attn_backward (see the module docstring)."""
    import torch

    from block_sparse_long_bigbird_amd import binding as bb
    from block_sparse_long_bigbird_amd.workloads import make_dout, make_inputs

    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    off, rows = bb.bb_rand_idx_invert(ri, w.H, w.L, w.block, w.r)
    inputs = make_inputs(w)
    dout = make_dout(w)
    q, k, v, pad = inputs
    dpad = None if pad is None else pad.to(dev)
    dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
    doff = torch.from_numpy(off).to(dev)
    drows = torch.from_numpy(rows).to(dev) if rows.size else None
    fws = bb.alloc_workspace(w.B, w.H, w.L, w.d, w.block, dev)
    dq0, dk0, dv0, dg0 = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    out0 = torch.empty_like(dq0)
    lse0 = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    qflag = bb.BB_QUERY_MASK if args.query_mask else 0
    bb.bb_attn_forward_lse(dq0, dk0, dv0, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, out0, fws, lse0,
                           flags=qflag)
    # cold mode: rotate among copies of the inputs (q, k, v, out, dout: 5 x 25 MB on the
    # headline shape) and outputs so that each call reads HBM
    footprint = 8 * dq0.numel() * dq0.element_size()
    n_sets = 1 if args.mode == "warm" else max(2, math.ceil(2.1 * LLC_BYTES / footprint))
    sets = []
    for i in range(n_sets):
        c = (lambda t: t) if i == 0 else (lambda t: t.clone())
        sets.append((c(dq0), c(dk0), c(dv0), c(out0), c(dg0), c(lse0),
                     torch.empty_like(dq0), torch.empty_like(dq0), torch.empty_like(dq0)))
    n = bb.bb_attn_backward_workspace_bytes(w.B, w.H, w.L, w.d, w.block)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call(i):
        a, b_, c, o, g, l, gq, gk, gv = sets[i % n_sets]
        bb.bb_attn_backward(a, b_, c, dpad, dri, doff, drows, w.B, w.H, w.L, w.d, w.block, w.r,
                            o, g, l, gq, gk, gv, ws, stream=stream.cuda_stream, flags=qflag)

    settle = settle_calls(args, "backward")
    for i in range(settle + args.warmup):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = 2.5 * useful_flops(w)
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": f"useful TFLOP/s, BigBird attn bwd{' (pair-masked)' if args.query_mask else ''} "
                  f"L={w.L} H={w.H} d={w.d} {w.dtype}, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) draws shaped like the BigBird-base attention layer)",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "L": w.L, "d": w.d,
                   "block": w.block, "r": w.r, "pad": w.pad, "mode": args.mode, "input_sets": n_sets,
                   "clock_settle_calls": settle,
                   "query_mask": bool(args.query_mask),
                   "useful_gflop_per_step": round(flops / 1e9, 4),
                   "executed_gflop_per_step": round(3.5 * useful_flops(w) / 1e9, 4)},
        "roofline": {"bound": "mfma", "kernel": "whole backward call (dq, dkdv, reduce)",
                     "achieved": round(value, 3), "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                     "frac": round(value / PEAK_TFLOPS[w.dtype], 4), "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(w, inputs, dout, ri, args.cpu_budget_s,
                                                    query_mask=args.query_mask)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 500 calls (~30 ms of kernels): the engine clock ramps up over the first
    # few milliseconds of load (a smaller W gets untimed clock-settle calls
    # first, CLOCK_SETTLE).
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=["cold", "warm"], default="cold")
    ap.add_argument("--launch", choices=["fused", "split"], default="fused")
    ap.add_argument("--query-mask", action="store_true",
                    help="forward with BB_QUERY_MASK (a pair is masked when its query or its key "
                         "is padding)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed passes, run a plain device copy of a known size "
                         "(reference point for the HBM byte counters)")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="after the timed passes, run a plain bf16 GEMM of a known size "
                         "(reference point for the MFMA counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--pmc-mfma-summary", metavar="COUNTER_CSV")
    ap.add_argument("--command", default="", help="profiling command recorded by --pmc-summary")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "layer", "stack"],
                    default="forward")
    ap.add_argument("--layers", type=int, default=12,
                    help="layers in the --pass stack call (BigBird-base has 12)")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, args.command)
        return
    if args.pmc_mfma_summary:
        pmc_mfma_summary(args.pmc_mfma_summary, args.workload, args.command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); (batch, head) units shard across GPUs with no "
              "communication, but no multi-GPU path is built here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_long_bigbird_amd import binding as bb
    from block_sparse_long_bigbird_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    bb.lib()
    if args.which == "backward":
        bench_backward(args, w, dev)
        return
    if args.which in ("layer", "stack"):
        bench_layer(args, w, dev, stack=args.which == "stack")
        return
    launch = bb.BB_LAUNCH_SPLIT if args.launch == "split" else bb.BB_LAUNCH_FUSED
    if args.query_mask:
        launch |= bb.BB_QUERY_MASK

    t0 = time.perf_counter()
    ri = bb.bb_rand_idx_build(w.rand_seed, w.H, w.L, w.block, w.r)
    t_adj = time.perf_counter() - t0
    inputs = make_inputs(w)
    q, k, v, pad = inputs
    es = 2 if w.dtype == "bf16" else 4
    footprint = 4 * w.B * w.H * w.L * w.d * es
    n_sets = 1 if args.mode == "warm" else max(2, math.ceil(2.1 * LLC_BYTES / footprint))
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    sets = [(dq, dk, dv, torch.empty_like(dq))]
    for _ in range(n_sets - 1):
        sets.append((dq.clone(), dk.clone(), dv.clone(), torch.empty_like(dq)))
    dpad = None if pad is None else pad.to(dev)
    dri = torch.from_numpy(ri).to(dev) if w.r > 0 else None
    ws = bb.alloc_workspace(w.B, w.H, w.L, w.d, w.block, dev)
    stream = torch.cuda.current_stream(dev)

    def call(i, flags, events=None):
        a, b_, c, o = sets[i % n_sets]
        bb.bb_attn_forward(a, b_, c, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, o, ws,
                           stream=stream.cuda_stream, flags=flags, events=events)

    # the timed calls: arguments checked once per input set (PreparedForward),
    # so a small problem's call is not bounded by the host-side checks
    prepared = [bb.PreparedForward(a, b_, c, dpad, dri, w.B, w.H, w.L, w.d, w.block, w.r, o, ws,
                                   stream=stream.cuda_stream, flags=launch) for a, b_, c, o in sets]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    settle = settle_calls(args, "forward")
    for i in range(settle + args.warmup):
        prepared[i % n_sets]()
    torch.cuda.synchronize()

    # Pass 1 -- the timed region: K whole steps, device synchronised on both sides.
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        prepared[i % n_sets]()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # Pass 2 -- per-kernel durations: the same steps in two phases, each
    # launch timestamped at its kernel's start and end by the launch itself
    # (bb_attn_forward_timed), on the launch stream.
    e = [(ev(), ev(), ev(), ev()) for _ in range(args.steps)]
    for x in e:                  # create the HIP events behind them
        for y in x:
            y.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        call(i, launch | bb.BB_PHASE_UNITS, events=(e[i][0], e[i][1]))
        call(i, launch | bb.BB_PHASE_MERGE, events=(e[i][2], e[i][3]))
    torch.cuda.synchronize()
    units_each = np.array([x[0].elapsed_time(x[1]) for x in e])
    units_ms = float(np.mean(units_each))
    merge_ms = float(np.mean([x[2].elapsed_time(x[3]) for x in e]))

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.mfma_calibration:
        # a plain bf16 GEMM of known size (torch.matmul): the reference point that
        # turns MFMA counter readings into FLOPs
        n = MFMA_CALIB_N
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
        torch.cuda.synchronize()
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()

    flops = useful_flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    alg_bytes = algorithmic_bytes(w)
    _, small = bb.bb_attn_forward_plan(w.B, w.H, w.L, w.d, w.block, w.r, w.dtype, launch)
    pre = "bb_sub32_" if w.dtype == "bf16" and w.block == 128 else "bb_"
    if small:
        kernel = "bb_small_kernel"
    elif args.launch == "fused":
        kernel = pre + "fused_kernel"
    else:
        kernel = f"{pre}global_rows_kernel+{pre}middle_rows_kernel"
    achieved = flops / (units_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = committed_traffic(w.name) if kernel == MAIN_KERNEL and not args.query_mask else None

    out = {
        "metric": METRIC if w.name == DEFAULT_WORKLOAD and not args.query_mask else
                  f"useful TFLOP/s + tokens/s, BigBird attn fwd{' (pair-masked)' if args.query_mask else ''} "
                  f"L={w.L} H={w.H} d={w.d} {w.dtype}, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "tokens_per_s": round(w.tokens / (ms_per_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) draws shaped like the BigBird-base attention layer)",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "block": w.block, "r": w.r,
            "pad": w.pad, "mode": args.mode, "input_sets": n_sets, "launch": args.launch,
            "clock_settle_calls": settle,
            "query_mask": bool(args.query_mask),
            "useful_gflop_per_step": round(flops / 1e9, 4),
            "algorithmic_mb_per_step": round(alg_bytes / 1e6, 3),
            "rand_idx_build_ms_host_untimed": round(t_adj * 1e3, 3),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "launch_us_mean": round(units_ms * 1e3, 3),
            "launch_us_p10_median_p90": [round(float(np.percentile(units_each, p)) * 1e3, 3) for p in (10, 50, 90)],
            "merge_us_mean": round(merge_ms * 1e3, 3),

            "hbm_algorithmic_GBps": round(alg_bytes / (units_ms * 1e-3) / 1e9, 1),
            "hbm_algorithmic_frac": round(alg_bytes / (units_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "cpu_baseline": None,
    }
    if traffic is not None:
        out["roofline"]["traffic_GBps"] = round(traffic / (units_ms * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inputs, ri, args.cpu_budget_s, query_mask=args.query_mask)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
