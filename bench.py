"""Throughput of the block-local MHSA sub-layer on one MI355X.

One step = one call of gs_block_mhsa_fwd (Q|K|V projection, block attention,
output projection with residual) over the whole packed batch, inputs already
resident in HBM.  Prints one JSON line.  The step time is the median over the
timed steps of the GPU time between HIP events recorded on the launch stream
at the step boundaries (K steps back to back, no events between a step's
kernels), with p10, p90, the mean and the wall-clock mean beside it.
Per-kernel times are means over a second pass of K steps in which the
library records events between the stages.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  python bench.py --copy-calibration MB   (plain device copy of MB MiB, for
                                           scaling HBM byte counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from conformer_block_attention_amd import accounting, gsattn, workloads  # noqa: E402

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
NOMINAL_CLOCK_MHZ = 2400.0  # the clock the published peaks are quoted at
KERNELS = ("qkv_proj", "block_attn", "out_proj")
HEADLINE_METRIC = "encoder frames/sec through block-MHSA (bf16, B=128 packed); % bf16 MFMA peak"
KERNEL_SOURCES = {
    "qkv_proj": ["gemm_bf16.hip", "gemm_pp_bf16.hip", "attn_units.hpp"],
    "out_proj": ["gemm_bf16.hip", "gemm_pp_bf16.hip", "attn_units.hpp"],
    "block_attn": ["attn_bf16.hip", "attn_units.hpp"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["gs_device.hpp"]:
        with open(os.path.join(ROOT, "conformer_block_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs of this
    workload (profiles/traffic_<kernel>.json for the headline batch,
    traffic_<kernel>.<workload>.json for others), if the kernel's sources are
    still those that were measured."""
    for name in (f"traffic_{kernel}.{workload}.json", f"traffic_{kernel}.json"):
        p = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(p):
            continue
        with open(p) as f:
            t = json.load(f)
        if t.get("workload", "").split(" ")[0] != workload:
            continue
        if t.get("source_hash") != source_hash(kernel):
            return None
        return t.get("bytes_per_launch")
    return None


def counters_for(kernel: str, workload: str, achieved_tflops: float):
    """MFMA busy fraction and average clock of the kernel's main launch from
    the committed rocprofv3 counter runs (profiles/counters_<kernel>.json),
    if its sources are still those that were measured, with the bf16 peak
    scaled to that clock and the achieved rate against it."""
    p = os.path.join(ROOT, "profiles", f"counters_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("workload", "").split(" ")[0] != workload or c.get("source_hash") != source_hash(kernel):
        return None
    peak = BF16_PEAK_TFLOPS * c["clock_mhz"] / NOMINAL_CLOCK_MHZ
    return {"kernel": kernel, "mfma_busy": c["mfma_busy"], "clock_mhz": c["clock_mhz"],
            "peak_at_clock": peak, "frac_at_clock": achieved_tflops / peak,
            "source": f"profiles/counters_{kernel}.json"}


def cpu_baseline(case, budget_s: float = 12.0):
    """The CPU oracle, untuned, on whole sequences of the workload in packing order
    until about `budget_s` seconds have passed."""
    import oracle

    orc = oracle.load()
    nthreads = oracle.host_threads()
    wqkv, wo = case.weights[0]
    w1, w2 = wqkv.double().numpy(), wo.double().numpy()
    frames = 0
    seqs = 0
    t0 = time.perf_counter()
    t = case.bucket_frames
    for s in range(len(case.lengths)):
        if t:  # one padded bucket
            xs = case.x[s * t:(s + 1) * t].double().numpy()
            orc.block_mhsa_padded(xs, case.lengths[s:s + 1], t, w1, w2, case.block_frames,
                                  case.heads, nthreads=nthreads)
            frames += int(case.lengths[s])
        else:
            a, b = int(case.cu[s]), int(case.cu[s + 1])
            xs = case.x[a:b].double().numpy()
            orc.block_mhsa(xs, np.array([0, b - a], np.int32), w1, w2, case.block_frames,
                           case.heads, nthreads=nthreads)
            frames += b - a
        seqs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": frames / el, "unit": "frames/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {seqs} of {len(case.lengths)} sequences ({frames} frames), "
                      f"one layer, fp64, {el:.1f} s"}


def cpu_baseline_xattn(c, budget_s: float = 12.0):
    """The window cross-attention oracle, untuned, window by window in order
    until about `budget_s` seconds have passed."""
    from oracle import window_xattn as wx

    t0 = time.perf_counter()
    nw = c.xq.shape[0]
    row0, lens = wx.window_table(c.cu, c.window_frames)
    wq, wkv, wo = (t.double().numpy() for t in (c.wq, c.wkv, c.wo))
    done = frames = 0
    step = 64
    while done < nw and time.perf_counter() - t0 < budget_s:
        ws = range(done, min(nw, done + step))
        # the windows [done, done + step) cover rows [a, b); a is a window
        # start, so cutting at a, b and the sequence starts between them
        # gives the same windows
        a = int(row0[ws[0]])
        b = int(row0[ws[-1]] + lens[ws[-1]])
        cut = sorted({a, b} | {int(v) for v in np.asarray(c.cu, np.int64) if a < v < b})
        sub_cu = np.asarray([v - a for v in cut], np.int64)
        wx.window_xattn(c.hcat[a:b].double().numpy(), sub_cu, c.xq[done:done + len(ws)].double().numpy(),
                        wq, wkv, wo, c.heads, c.window_frames)
        frames += b - a
        done += len(ws)
    el = time.perf_counter() - t0
    try:  # the oracle's matrix products run on numpy's BLAS threads
        import threadpoolctl
        cores = max([p["num_threads"] for p in threadpoolctl.threadpool_info()
                     if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        cores = None
    return {"value": frames / el, "unit": "frames/s", "cores": cores,
            "kind": "oracle", "sample": f"first {done} of {nw} windows ({frames} frames), fp64, "
                                        f"{el:.1f} s"}


def time_steps(step, steps: int, stream):
    """GPU milliseconds of each of `steps` calls of step() run back to back,
    from HIP events recorded on `stream` at the step boundaries only (an
    event between two kernels leaves the GPU idle for about 6 us on this
    chip, which no caller pays), and the wall-clock seconds of the run."""
    bev = gsattn.HipEvents(steps + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bev.record(0, stream)
    for k in range(steps):
        step()
        bev.record(k + 1, stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return np.array([bev.elapsed_ms(k, k + 1) for k in range(steps)]), el


def _hwmon_power_file():
    """The GPU's board-power reading in sysfs (microwatts), if there is one."""
    import glob
    for pat in ("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input",
                "/sys/class/drm/card*/device/hwmon/hwmon*/power1_average"):
        for f in sorted(glob.glob(pat)):
            try:
                with open(f) as fh:
                    int(fh.read().strip())
                return f
            except (OSError, ValueError):
                continue
    return None


def board_power(step, seconds: float = 3.0, settle: float = 1.0):
    """Mean board power while step() runs back to back for `seconds`: the
    hwmon reading sampled every 20 ms by a thread, after `settle` seconds in
    which the board ramps up from idle.  None if no reading is available."""
    import threading

    f = _hwmon_power_file()
    if f is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.perf_counter()
        while not stop.is_set():
            if time.perf_counter() - t0 >= settle:
                try:
                    with open(f) as fh:
                        samples.append(int(fh.read().strip()) / 1e6)
                except (OSError, ValueError):
                    pass
            time.sleep(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"mean": float(np.mean(samples)), "max": float(np.max(samples)),
            "samples": len(samples), "window_s": seconds - settle, "source": f}


def bench_xattn(args):
    """The window cross-attention of the Q-Former projector on its workload."""
    w = workloads.XATTN_WORKLOADS[args.workload]
    c = workloads.build_xattn_case(w)
    dev = torch.device("cuda:0")
    hcat, xq = c.hcat.to(dev), c.xq.to(dev)
    cu = torch.from_numpy(c.cu).to(dev)
    wq, wkv, wo = c.wq.to(dev), c.wkv.to(dev), c.wo.to(dev)
    n, f = hcat.shape
    nw, nq, dq = xq.shape
    lib = gsattn.load()
    ws = torch.empty(lib.gs_window_xattn_workspace_bytes(n, dq, nw, nq), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(xq)
    stream = torch.cuda.current_stream()

    def step(events=None, base=0):
        gsattn.window_xattn_fwd(hcat, cu, xq, wq, wkv, wo, c.window_frames, c.heads, out=out,
                                workspace=ws, stream=stream,
                                kernel_events=events.view(base) if events else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ms, el = time_steps(step, args.steps, stream)
    # per-kernel durations: a second pass with the library's stage events
    ev = gsattn.HipEvents(4 * args.steps)
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(ev, 4 * k)
    torch.cuda.synchronize()
    names = ("kv_q_proj", "window_attn", "out_proj")
    avg = {k: float(np.mean([ev.elapsed_ms(4 * i + j, 4 * i + j + 1) for i in range(args.steps)]))
           for j, k in enumerate(names)}
    rows = nw * nq
    fl = {"kv_q_proj": 2.0 * n * f * 2 * dq + 2.0 * rows * dq * dq,
          "window_attn": 4.0 * nq * n * dq,
          "out_proj": 2.0 * rows * dq * dq}
    by = {"kv_q_proj": 2 * (n * f + 2 * dq * f + 2 * n * dq + 2 * rows * dq + dq * dq),
          "window_attn": 2 * (2 * n * dq + 2 * rows * dq),
          "out_proj": 2 * (3 * rows * dq + dq * dq)}
    dom = max(avg, key=avg.get)
    if by[dom] / (HBM_PEAK_GBS * 1e9) > fl[dom] / (BF16_PEAK_TFLOPS * 1e12):
        a = by[dom] / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS}
    else:
        a = fl[dom] / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": a, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a / BF16_PEAK_TFLOPS}
    roof["kernel"] = dom
    roof["traffic"] = None
    total = sum(fl.values())
    p10, p50, p90 = (float(v) for v in np.percentile(step_ms, [10, 50, 90]))
    sec = p50 * 1e-3
    rec = {
        "metric": f"encoder frames/sec through the window cross-attention ({w.name}); "
                  f"% of matrix peak",
        "value": n / sec, "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec * 1e3,
        "step_ms": {"median": p50, "p10": p10, "p90": p90, "mean": float(np.mean(step_ms)),
                    "wall_mean": el / args.steps * 1e3},
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "global_batch": int(len(c.lengths)), "frames": int(n),
                   "windows": int(nw), "queries": nq, "feat_dim": int(f), "d_q": int(dq),
                   "heads": c.heads, "window_frames": c.window_frames, "seed": w.seed},
        "tflops": total / sec / 1e12, "pct_bf16_peak": 100.0 * total / sec / 1e12 / BF16_PEAK_TFLOPS,
        "useful_gflop": total / 1e9,
        "kernels": {k: {"avg_ms": avg[k], "tflops": fl[k] / (avg[k] * 1e-3) / 1e12,
                        "alg_GBs": by[k] / (avg[k] * 1e-3) / 1e9} for k in names},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_xattn(c, args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


CTC_WORKLOAD = "bpe_pool_ctc_b128"


def bench_ctc(args):
    """Posterior-weighted pooling + CTC greedy decoding of the BPE head's
    logits for the headline batch's frames (HBM-bound: the logits are read
    once)."""
    lengths = workloads.WORKLOADS[workloads.HEADLINE].lengths()
    logits, bp, cu = workloads.bpe_inputs(lengths)
    n, ld = logits.shape
    classes = workloads.BPE_CLASSES
    lib = gsattn.load()
    npos = int(np.sum((lengths + 1) // 2))
    dev = logits.device
    out = (torch.empty(npos, dtype=torch.int32, device=dev),
           torch.empty(npos, dtype=torch.int32, device=dev),
           torch.empty(len(lengths), dtype=torch.int32, device=dev))
    ws = torch.empty(lib.gs_bpe_ctc_workspace_bytes(len(lengths), npos), dtype=torch.uint8,
                     device=dev)

    def step():
        gsattn.bpe_pool_ctc_greedy(logits, bp, cu, classes, npos, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ms, el = time_steps(step, args.steps, torch.cuda.current_stream())
    p10, ms, p90 = (float(v) for v in np.percentile(step_ms, [10, 50, 90]))
    by = 2 * n * ld + 4 * n + 8 * npos + 4 * len(lengths)  # logits, blank probs, outputs
    gbs = by / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ctc_pool as cp
        t1 = time.perf_counter()
        cuh = workloads.cu_seqlens(lengths)
        frames = seqs = 0
        while seqs < len(lengths) and time.perf_counter() - t1 < args.cpu_budget:
            a, b = int(cuh[seqs]), int(cuh[seqs + 1])
            ids = cp.pooled_argmax(logits[a:b, :classes].float().cpu().numpy(),
                                   bp[a:b].cpu().numpy(), [0, b - a])
            cp.ctc_greedy(ids, [len(ids)])
            frames += b - a
            seqs += 1
        ce = time.perf_counter() - t1
        cpu = {"value": frames / ce, "unit": "frames/s", "cores": 1, "kind": "oracle",
               "sample": f"first {seqs} of {len(lengths)} sequences ({frames} frames), "
                         f"{ce:.1f} s (includes copying their logits to the host)"}
    rec = {
        "metric": f"encoder frames/sec through BPE pooling + CTC greedy decoding ({CTC_WORKLOAD}); "
                  f"% of HBM peak",
        "value": n / (ms * 1e-3), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms,
        "step_ms": {"median": ms, "p10": p10, "p90": p90, "mean": float(np.mean(step_ms)),
                    "wall_mean": el / args.steps * 1e3},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CTC_WORKLOAD, "global_batch": int(len(lengths)), "frames": int(n),
                   "positions": npos, "classes": classes, "ld": int(ld), "window": 4,
                   "stride": 2},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "kernel": "pooled_argmax + collapse",
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


# kernel roles by name (rocprofv3 reports template arguments in the name)
KERNEL_ROLES = (
    ("gemm_pp_bf16_kernel<256, false", "qkv_proj"),
    ("gemm_pp_bf16_kernel<256, true", "out_proj"),
    ("gemm_bf16_nt_kernel<64, 128, 64, 3, false, 0, 4, false>", "qkv_proj (last rows)"),
    ("gemm_bf16_nt_kernel<192, 128, 64, 3, false, 0, 4, true>", "out_proj (last rows)"),
    ("block_attn_bf16_kernel", "block_attn"),
    ("build_unit_table_kernel", "(attention work-unit table)"),
)
CUS, SIMDS_PER_CU, XCDS = 256, 4, 8


def _role(kernel_name: str) -> str:
    for key, role in KERNEL_ROLES:
        if key in kernel_name:
            return role
    return kernel_name.split("(")[0]


def counter_summary(outdir: str) -> dict:
    """Per-kernel averages of the counters in rocprofv3's CSV output under
    `outdir` (any *counter_collection.csv, joined by dispatch to the
    *kernel_trace.csv beside it), with derived figures.  rocprofv3 sums a
    counter over its hardware instances, so GRBM_GUI_ACTIVE comes as the sum
    of the 8 XCDs' active cycles; per XCD it is the kernel's cycle count:
      cycles      = GRBM_GUI_ACTIVE / 8
      clock_mhz   = cycles / duration
      mfma_busy   = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)
                    (the busy count is summed over SIMDs; a 32x32x16 bf16
                    product counts 32 cycles, a 16x16x32 one 16)
      mfma_flop   = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
      lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
    GRBM_GUI_ACTIVE also counts a few microseconds around each dispatch, so
    the clock of a kernel much shorter than 100 us reads high."""
    import csv
    import glob

    dur = {}
    for f in glob.glob(os.path.join(outdir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur[(f.rsplit("kernel_trace.csv", 1)[0], r["Dispatch_Id"])] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    acc = {}
    for f in glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True):
        pre = f.rsplit("counter_collection.csv", 1)[0]
        for r in csv.DictReader(open(f)):
            k = _role(r["Kernel_Name"])
            e = acc.setdefault(k, {"dispatches": set(), "ns": {}, "counters": {}})
            did = r["Dispatch_Id"]
            e["dispatches"].add((pre, did))
            if (pre, did) in dur:
                e["ns"][(pre, did)] = dur[(pre, did)]
            c = e["counters"].setdefault(r["Counter_Name"], {})
            c[(pre, did)] = c.get((pre, did), 0.0) + float(r["Counter_Value"])
    out = {}
    for k, e in acc.items():
        avg = {n: sum(v.values()) / len(v) for n, v in e["counters"].items()}
        rec = {"dispatches": len(e["dispatches"]), "counters": avg}
        if e["ns"]:
            rec["avg_us"] = sum(e["ns"].values()) / len(e["ns"]) / 1e3
        g = avg.get("GRBM_GUI_ACTIVE")
        if g:
            rec["cycles"] = g / XCDS
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            rec["mfma_busy"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / XCDS * CUS * SIMDS_PER_CU)
        if g and e["ns"]:
            # per-dispatch ratio of active cycles to nanoseconds
            ratios = [e["counters"]["GRBM_GUI_ACTIVE"][d] / XCDS / e["ns"][d]
                      for d in e["ns"] if d in e["counters"]["GRBM_GUI_ACTIVE"] and e["ns"][d]]
            rec["clock_mhz"] = 1e3 * sum(ratios) / len(ratios)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            rec["mfma_flop"] = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            rec["lds_conflict"] = avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / avg["SQ_LDS_IDX_ACTIVE"]
        out[k] = rec
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=workloads.HEADLINE,
                    choices=workloads.WORKLOAD_ORDER + list(workloads.XATTN_WORKLOADS) +
                    [CTC_WORKLOAD])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the 3 s pass that reads the board power")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB MiB, 5 times")
    ap.add_argument("--counter-summary", default="", metavar="DIR",
                    help="only summarise the rocprofv3 counter CSVs under DIR (no GPU)")
    args = ap.parse_args()

    if args.counter_summary:
        print(json.dumps(counter_summary(args.counter_summary), indent=1, sort_keys=True))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the sub-layer shards by whole sequences with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        # Reference kernel for the byte counters: reads and writes exactly
        # `nbytes` per launch.
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)
        return

    if args.workload in workloads.XATTN_WORKLOADS:
        bench_xattn(args)
        return
    if args.workload == CTC_WORKLOAD:
        bench_ctc(args)
        return
    w = workloads.WORKLOADS[args.workload]
    case = workloads.build_case(w, layers=w.layers)
    dev = torch.device("cuda:0")
    x = case.x.to(dev)
    cu = torch.from_numpy(case.cu).to(dev)
    weights = [(a.to(dev), b.to(dev)) for a, b in case.weights]
    n, d = x.shape
    nl = len(weights)
    if case.bucket_frames:
        nb = gsattn.load().gs_block_mhsa_padded_workspace_bytes(
            len(case.lengths), case.bucket_frames, d, gsattn._gs_dtype(x.dtype))
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    else:
        ws = gsattn.alloc_workspace(n, d, x.dtype, dev)
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    stream = torch.cuda.current_stream()

    t = case.bucket_frames
    lens = torch.from_numpy(case.lengths.astype(np.int32)).to(dev)

    def step(events=None, ev_base=0):
        cur = x
        for l, (wqkv, wo) in enumerate(weights):
            o = bufs[l & 1]
            kev = events.view(ev_base + 4 * l) if events else None
            if t:
                gsattn.block_mhsa_fwd_padded(cur.view(-1, t, d), lens, wqkv, wo, case.block_frames,
                                             case.heads, out=o.view(-1, t, d), workspace=ws,
                                             stream=stream, kernel_events=kev)
            else:
                # a stack of layers over one batch builds the attention's
                # work-unit table once, in its first layer
                gsattn.block_mhsa_fwd(cur, cu, wqkv, wo, case.block_frames, case.heads, out=o,
                                      workspace=ws, stream=stream, kernel_events=kev,
                                      reuse_unit_table=l > 0)
            cur = o
        return cur

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # step timing: K steps back to back, events at the step boundaries only
    step_ms, el = time_steps(step, args.steps, stream)

    # Kernel timing: K more steps with the library's events between the
    # stages, for the per-kernel durations.
    ev = gsattn.HipEvents(4 * nl * args.steps)
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(ev, 4 * nl * k)
    torch.cuda.synchronize()

    power = None if args.no_power else board_power(step)

    per = {k: [] for k in KERNELS}
    for i in range(nl * args.steps):
        b = 4 * i
        per["qkv_proj"].append(ev.elapsed_ms(b, b + 1))
        per["block_attn"].append(ev.elapsed_ms(b + 1, b + 2))
        per["out_proj"].append(ev.elapsed_ms(b + 2, b + 3))
    avg_ms = {k: float(np.mean(v)) for k, v in per.items()}
    p10, p50, p90 = (float(v) for v in np.percentile(step_ms, [10, 50, 90]))

    ms_step = p50
    valid = int(np.sum(case.lengths))  # frames (padding rows excluded)
    frames_per_s = valid * nl / (ms_step * 1e-3)  # frame-layers per second
    fl = accounting.useful_flops(case.lengths, d, case.block_frames)
    tflops = fl["total"] * nl / (ms_step * 1e-3) / 1e12
    bf16 = x.dtype == torch.bfloat16
    peak = BF16_PEAK_TFLOPS if bf16 else F32_PEAK_TFLOPS
    elem = 2 if bf16 else 4
    by = accounting.algorithmic_bytes(n, d, elem)  # all rows the projections touch
    if t:  # padded: attention reads Q|K|V of the valid rows and writes O for every row
        by["block_attn"] = elem * (3 * valid * d + n * d)

    # dominant kernel and its roofline: the bound is whichever of its useful
    # flops at the matrix peak and its algorithmic bytes at the HBM peak takes
    # longer (the attention of 200-frame blocks is HBM-bound, that of whole
    # sequences of thousands of frames is not)
    dom = max(avg_ms, key=avg_ms.get)
    if by[dom] / (HBM_PEAK_GBS * 1e9) > fl[dom] / (peak * 1e12):
        achieved = by[dom] / (avg_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = fl[dom] / (avg_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof["kernel"] = dom
    roof["traffic"] = traffic_for(dom, w.name) if bf16 else None

    kernels = {}
    for k in KERNELS:
        kernels[k] = {"avg_ms": avg_ms[k],
                      "tflops": fl[k] / (avg_ms[k] * 1e-3) / 1e12,
                      "alg_GBs": by[k] / (avg_ms[k] * 1e-3) / 1e9}

    rec = {
        "metric": (HEADLINE_METRIC if w.name == workloads.HEADLINE else
                   f"encoder frames/sec through block-MHSA ({w.name}); % of matrix peak"),
        "value": frames_per_s,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"median": p50, "p10": p10, "p90": p90, "mean": float(np.mean(step_ms)),
                    "wall_mean": el / args.steps * 1e3},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": int(len(case.lengths)), "frames": valid,
                   "rows": int(n), "bucket_frames": t or None,
                   "blocks": len(accounting.block_table(case.lengths, case.block_frames)),
                   "block_frames": case.block_frames, "d_model": int(d), "heads": case.heads,
                   "layers": nl, "seed": w.seed},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / peak,
        "useful_gflop_per_layer": fl["total"] / 1e9,
        "kernels": kernels,
        "roofline": roof,
        "counters": (counters_for(dom, w.name, fl[dom] / (avg_ms[dom] * 1e-3) / 1e12)
                     if bf16 else None),
        # board power while the step runs back to back (hwmon, after a 1 s
        # ramp), and the energy of one step at that power
        "board_power_w": (dict(power, joules_per_step=power["mean"] * ms_step * 1e-3)
                          if power else None),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
