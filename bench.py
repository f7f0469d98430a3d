#!/usr/bin/env python3
"""Throughput of the fused LM-head cross-entropy forward+backward on one MI355X.

One step = one fldce_fwd_bwd call over the whole batch: logits GEMM with the
softmax-partials epilogue, per-row combine and loss, dlogits, dH = g W,
dW = g^T h and the loss reduction (every stage of the path), with inputs,
outputs and workspace resident in HBM before the timed region starts.

Default workload: the headline masked-diffusion LM head, B=8 x L=1024
(N=8192 tokens), H=2560, V=151936, bf16, label_smoothing 0.1, logit_scale
0.5, per-sequence masking probability, mean over N ("sum/N").  Synthetic,
seeded inputs (lm_head_linear_bf16_amd.synth).

Prints ONE JSON line: tokens/s (value; all N tokens), executed TFLOP/s
(6 * rows multiplied * H * V: the bf16 path multiplies only rows whose target
is not ignore_index, the rest are exactly zero) and its fraction of the bf16
MFMA peak, the dense-equivalent 6*N*H*V rate, the roofline entry of the dominant kernel (timed live with
HIP events recorded on the library's stream inside the timed steps), and the
float64 CPU oracle timed on a bounded row sample on this host.

    python bench.py [--steps K] [--warmup W] [--workload headline] [--chunk-rows C]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector, published
# GEMM stages and their flops per step in units of rows * H * V: dH and dW
# are one launch ("bwd_gemms") when both are computed
STAGE_FLOP_KERNELS = {"logits_gemm": 2, "dH_gemm": 2, "dW_gemm": 2, "bwd_gemms": 4}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash() -> str:
    d = hashlib.sha256()
    cdir = os.path.join(ROOT, "lm_head_linear_bf16_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, name), "rb") as f:
            d.update(name.encode())
            d.update(f.read())
    return d.hexdigest()[:16]


def traffic_entry(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("src_hash") != src_hash():
        return None
    return e.get("bytes_per_launch")


def _counter_per_kernel(path: str, counter: str) -> dict:
    """{kernel short name: [value per dispatch (KiB)]} from a rocprofv3 counter CSV."""
    import csv
    out: dict = {}
    per_dispatch: dict = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    for (_, name), v in sorted(per_dispatch.items(), key=lambda kv: int(kv[0][0])):
        out.setdefault(name, []).append(v)
    return out


# the kernel instance each stage launches: plain fwd+bwd, and for the vocab
# shard workload the shard partials and the shard backward
STAGE_KERNELS = {"logits_gemm": "k_logits_bf16<1, 1, false>", "dH_gemm": "k_gemm_dh_bf16",
                 "dW_gemm": "k_gemm_dw_bf16<0>"}
SHARD_STAGE_KERNELS = {"partials_logits": "k_logits_bf16<0, 0, false>",
                       "bwd_logits": "k_logits_bf16<2, 1, false>", "dH_gemm": "k_gemm_dh_bf16",
                       "dW_gemm": "k_gemm_dw_bf16<0>"}
XCDS = 8  # MI355X: GRBM_GUI_ACTIVE is reported summed over the 8 XCDs' instances


WORKLOAD_NAMES = ("tiny", "4b", "headline", "block", "shard")


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, calib_mib: int,
                    cmd: str = "") -> int:
    """FETCH_SIZE / WRITE_SIZE per launch of each stage kernel, scaled by the
    ratio of the calibration copy's known bytes to what the same counter read
    for it; writes profiles/traffic.json and profiles/<workload>_traffic.md."""
    fetch = _counter_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _counter_per_kernel(write_csv, "WRITE_SIZE")
    calib = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not calib:
        print("no calibration copy kernel found in the counter file", file=sys.stderr)
        return 1
    known_kib = calib_mib * 1024.0
    cf = known_kib / max(fetch[calib[0]])
    cw = known_kib / max(write[calib[0]])
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            everything = json.load(f)
    except (OSError, ValueError):
        everything = {}
    everything = {k: v for k, v in everything.items() if k in WORKLOAD_NAMES}
    out = {}
    lines = [f"# HBM traffic per launch, {workload} workload",
             "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs,",
             "one with FETCH_SIZE and one with WRITE_SIZE (each beside one more TCC counter),",
             "",
             f"    {cmd or 'rocprofv3 --kernel-trace --pmc <counters> -- python3 bench.py --workload ' + workload + ' --steps 2 --warmup 1 --no-cpu-baseline --no-extras --sweep= --calib-copy-mib ' + str(calib_mib)}",
             "",
             f"scaled by the calibration copy of {calib_mib} MiB (read scale {cf:.4f}, write scale {cw:.4f}).",
             "",
             "| stage | kernel | fetch GB/launch | write GB/launch | launches |",
             "|---|---|---|---|---|"]
    kernels = SHARD_STAGE_KERNELS if workload == "shard" else STAGE_KERNELS
    for stage, kname in kernels.items():
        fk = [k for k in fetch if kname in k]
        wk = [k for k in write if kname in k]
        if not fk or not wk:
            continue
        fv = [v for k in fk for v in fetch[k]]
        wv = [v for k in wk for v in write[k]]
        fb = sum(fv) / len(fv) * 1024 * cf
        wb = sum(wv) / len(wv) * 1024 * cw
        out[stage] = {"kernel": kname, "src_hash": src_hash(), "fetch_bytes": fb,
                      "write_bytes": wb, "bytes_per_launch": fb + wb, "launches": len(fv),
                      "read_scale": cf, "write_scale": cw}
        lines.append(f"| {stage} | {kname} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {len(fv)} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    everything[workload] = out
    with open(path, "w") as f:
        json.dump(everything, f, indent=1)
    with open(os.path.join(ROOT, "profiles", f"{workload}_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def _durations(trace_csv: str) -> dict:
    """{dispatch id: kernel duration in ns} from a rocprofv3 kernel-trace CSV."""
    import csv
    out = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            out[r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def counter_summary(run_dirs, workload: str, cmd: str, calib_mib: int) -> int:
    """Per stage kernel, averages over its launches of the counters of several
    rocprofv3 --pmc --kernel-trace runs (one directory each): the average
    shader clock (GRBM_GUI_ACTIVE cycles over the launch's duration), MFMA
    busy (SQ_VALU_MFMA_BUSY_CYCLES over 4 SIMDs x 256 CUs x those cycles),
    VALU busy (SQ_ACTIVE_INST_VALU over 256 CUs x cycles, rocprofv3's VALUBusy),
    LDS active (SQ_LDS_IDX_ACTIVE over 256 CUs x cycles), the MFMA bf16 work,
    the L2's fetch and write bytes, and the bytes of the requests it sent to
    local HBM addresses, each scaled by what the same counter read for the
    calibration copy.  Writes profiles/<workload>_counters.md."""
    import csv
    import glob
    vals: dict = {}     # (kernel, counter) -> [per-dispatch values]
    durs: dict = {}     # kernel -> [ns]
    for d in run_dirs:
        cc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        kt = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
        if not cc:
            print(f"no counter CSV under {d}", file=sys.stderr)
            return 1
        dur = _durations(kt[0]) if kt else {}
        per: dict = {}
        names: dict = {}
        for path in cc:
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = (r["Dispatch_Id"], r["Counter_Name"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                    names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for (disp, cname), v in per.items():
            vals.setdefault((names[disp], cname), []).append(v)
        if "GRBM_GUI_ACTIVE" in {c for (_, c) in per}:
            for disp, name in names.items():
                if disp in dur:
                    durs.setdefault(name, []).append(dur[disp])
    avg = lambda xs: sum(xs) / len(xs) if xs else float("nan")  # noqa: E731
    # FETCH_SIZE / WRITE_SIZE scaled by what they read for the calibration copy
    # of calib_mib MiB (the run's first device copy)
    scale = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum"):
        cal = [v for (k, c), v in vals.items() if c == cname and
               ("copy" in k.lower() or "elementwise" in k.lower())]
        scale[cname] = calib_mib * 1024.0 / max(cal[0]) if cal and calib_mib else 1.0
    kernels = SHARD_STAGE_KERNELS if workload == "shard" else STAGE_KERNELS
    lines = [f"# Counters per launch of the stage kernels, {workload} workload", "",
             "rocprofv3 --pmc runs with --kernel-trace (one counter group per run), each", "",
             f"    {cmd}", "",
             "clock = GRBM_GUI_ACTIVE / (8 XCDs x launch duration) (the counter is summed over "
             "the 8 XCDs' instances; a device copy reads 2.4 GHz this way); MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) (rocprofv3's MfmaUtil); VALU busy = "
             "SQ_ACTIVE_INST_VALU / (256 CUs x GRBM_GUI_ACTIVE) (rocprofv3's VALUBusy); LDS "
             "active = SQ_LDS_IDX_ACTIVE / (256 CUs x GRBM_GUI_ACTIVE) (rocprofv3's LdsUtil); "
             "MFMA TFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; fetch / write = FETCH_SIZE / "
             "WRITE_SIZE, each scaled by what it read for "
             f"a {calib_mib} MiB device copy (read x {scale['FETCH_SIZE']:.3f}, write x "
             f"{scale['WRITE_SIZE']:.3f}); HBM read / write = TCC_EA0_RDREQ_DRAM / "
             "TCC_EA0_WRREQ_DRAM (L2 requests to local HBM addresses) times the bytes per "
             f"request of the same copy ({scale['TCC_EA0_RDREQ_DRAM_sum'] * 1024:.0f} B read, "
             f"{scale['TCC_EA0_WRREQ_DRAM_sum'] * 1024:.0f} B write); the memory-side cache "
             "(MALL) may serve some of those requests, and no counter here separates its hits.", "",
             "| stage | kernel | launches | ms | clock GHz | MFMA busy % | MFMA TFLOP/s | "
             "VALU busy % | LDS active % | fetch GB | write GB | HBM read GB | HBM write GB | "
             "HBM GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for stage, kname in kernels.items():
        ks = [k for (k, _) in vals if kname in k]
        if not ks:
            continue
        k = ks[0]
        g = lambda c: avg(vals.get((k, c), []))  # noqa: E731
        gui = g("GRBM_GUI_ACTIVE") / XCDS  # cycles of one XCD
        ms = avg(durs.get(k, [])) * 1e-6
        clock = gui / (ms * 1e6) if ms == ms and ms > 0 else float("nan")
        mfma = 100.0 * g("SQ_VALU_MFMA_BUSY_CYCLES") / (1024.0 * gui)
        valu = 100.0 * g("SQ_ACTIVE_INST_VALU") / (256.0 * gui)
        lds = 100.0 * g("SQ_LDS_IDX_ACTIVE") / (256.0 * gui)
        tf = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512.0 / (ms * 1e-3) / 1e12
        fetch = g("FETCH_SIZE") * 1024 * scale["FETCH_SIZE"] / 1e9
        write = g("WRITE_SIZE") * 1024 * scale["WRITE_SIZE"] / 1e9
        hr = g("TCC_EA0_RDREQ_DRAM_sum") * 1024 * scale["TCC_EA0_RDREQ_DRAM_sum"] / 1e9
        hw = g("TCC_EA0_WRREQ_DRAM_sum") * 1024 * scale["TCC_EA0_WRREQ_DRAM_sum"] / 1e9
        lines.append(f"| {stage} | {kname} | {len(durs.get(k, []))} | {ms:.3f} | {clock:.2f} | "
                     f"{mfma:.1f} | {tf:.0f} | {valu:.1f} | {lds:.1f} | {fetch:.2f} | {write:.2f} | "
                     f"{hr:.2f} | {hw:.2f} | {(hr + hw) / (ms * 1e-3):.0f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{workload}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, rows: int) -> dict:
    """The float64 oracle on the first `rows` token rows of the same workload
    (all of them by default: one full call)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    import oracle
    from lm_head_linear_bf16_amd import synth
    target, p_mask = synth.targets(w)
    h = synth.hidden(w).values[:rows].astype(np.float64)
    W = synth.weight(w).values.astype(np.float64)
    t = target[:rows]
    p = p_mask[:rows]
    log(f"cpu baseline: oracle on {rows} rows, {threads} BLAS threads")
    t0 = time.perf_counter()
    oracle.forward_backward(h, W, t, p, label_smoothing=w.label_smoothing,
                            logit_scale=w.logit_scale, reduction=w.reduction,
                            total=w.total or None, row_block=1024)
    dt = time.perf_counter() - t0
    what = (f"the whole workload, all {w.N} token rows: one full call" if rows == w.N else
            f"first {rows} of {w.N} token rows of the same workload")
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} (full vocabulary; loss, dH, dW), float64 NumPy, {dt:.2f} s",
            "seconds": dt, "cpu_model": cpu_model(),
            "host_threads": len(os.sched_getaffinity(0))}


def env_info(torch) -> dict:
    """Device, HIP runtime and PyTorch versions of the run."""
    p = torch.cuda.get_device_properties(0)
    env = {"device": p.name, "arch": getattr(p, "gcnArchName", ""),
           "compute_units": p.multi_processor_count, "hip": torch.version.hip,
           "torch": torch.__version__}
    # the rated shader clock and L2 size, where this PyTorch build exposes them
    # (the clock a kernel actually runs at is in the counter summaries)
    clock_khz = getattr(p, "clock_rate", None)
    if clock_khz:
        env["max_clock_mhz"] = round(clock_khz / 1000.0)
    l2 = getattr(p, "L2_cache_size", None)
    if l2:
        env["l2_cache_mb"] = round(l2 / 2**20, 1)
    return env


def _timed(fn, steps: int, warmup: int):
    """(ms per call, {stage: ms per call}) with the library's stage events."""
    import torch
    from lm_head_linear_bf16_amd import fldce
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    fldce.fldce_profile_begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fldce.fldce_profile_end()
    stages = {}
    for st in range(fldce.fldce_profile_num_stages()):
        tot, n = fldce.fldce_profile_read(st)
        if n:
            stages[fldce.fldce_profile_stage_name(st)] = round(tot / steps, 4)
    return (t1 - t0) * 1e3 / steps, stages


def vendor_leg(w, rows: int, peak: float, reps: int = 10) -> dict:
    """For scale, not part of the path: torch.matmul (hipBLASLt) as plain bf16
    GEMMs at the three contractions' shapes of this workload, with the
    operands in the layouts the fused kernels read (rows = the rows with a
    target): logits W [V, H] x h [rows, H]^T, dH E [rows, V] x W [V, H], dW
    as its transpose h^T [H, rows] x E [rows, V].  Random operands; the
    median of `reps` timed calls per shape."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    H, V = w.H, w.V
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16
    Wm = torch.randn(V, H, device=dev, dtype=bf, generator=g)
    hm = torch.randn(rows, H, device=dev, dtype=bf, generator=g)
    Em = torch.randn(rows, V, device=dev, dtype=bf, generator=g)
    hT = hm.t().contiguous()
    shapes = {"logits": (lambda: torch.matmul(Wm, hm.t()), 2.0 * V * rows * H),
              "dH": (lambda: torch.matmul(Em, Wm), 2.0 * rows * V * H),
              "dW": (lambda: torch.matmul(hT, Em), 2.0 * H * rows * V)}
    out = {}
    for name, (fn, flops) in shapes.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
        log(f"vendor GEMM {name}: {ms:.3f} ms, {tf:.0f} TFLOP/s")
    del Wm, hm, Em, hT
    return out


def extra_legs(args, w, h, W, tgt, pm, dt, rows_mult: int, ms_plain: float, peak: float) -> dict:
    """The rest of page 1's interface on the same inputs: forward only
    (fldce_fwd: 2 * rows * H * V flops), with --frozen-leg fwd+bwd without
    dW, and with --bias-leg fwd+bwd with the seeded bias and its gradient db
    (fldce_fwd_bwd_ex)."""
    import numpy as np
    import torch
    from lm_head_linear_bf16_amd import fldce, synth
    N, H, V = w.N, w.H, w.V
    dev = h.device
    steps, warm = max(3, args.steps // 2), 1
    out = {}
    ws = torch.empty(fldce.fldce_fwd_workspace_size(N, H, V, dt), dtype=torch.uint8, device=dev)
    kw = dict(label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
              reduction=w.reduction, total=w.total)
    log(f"forward only: {steps} steps")
    m, st = _timed(lambda: fldce.fldce_fwd(h, W, tgt, pm, workspace=ws, **kw), steps, warm)
    tf = 2.0 * rows_mult * H * V / (m * 1e-3) / 1e12
    out["forward_only"] = {"ms_per_step": round(m, 4), "tokens_per_s": round(N / (m * 1e-3), 1),
                           "tflops": round(tf, 2), "pct_peak": round(100.0 * tf / peak, 2),
                           "stage_ms_per_step": st}
    del ws
    if args.frozen_leg:
        # a frozen LM-head weight: dH only (fldce_fwd_bwd_ex without dW), 4 * rows * H * V
        ws = torch.empty(fldce.fldce_workspace_size(N, H, V, dt), dtype=torch.uint8, device=dev)
        log(f"fwd+bwd without dW: {steps} steps")
        m, st = _timed(lambda: fldce.fldce_fwd_bwd_ex(h, W, tgt, pm, want_dW=False, workspace=ws,
                                                      **kw), steps, warm)
        tf = 4.0 * rows_mult * H * V / (m * 1e-3) / 1e12
        out["frozen_weight"] = {"ms_per_step": round(m, 4),
                                "tokens_per_s": round(N / (m * 1e-3), 1), "tflops": round(tf, 2),
                                "pct_peak": round(100.0 * tf / peak, 2), "stage_ms_per_step": st}
        del ws
    if not args.bias_leg:
        return out
    bt = synth.bias(w)
    b = (torch.from_numpy(bt.bits.view(np.int16)).view(torch.bfloat16) if bt.bits is not None
         else torch.from_numpy(bt.values)).to(dev)
    ws = torch.empty(fldce.fldce_workspace_size(N, H, V, dt), dtype=torch.uint8, device=dev)
    log(f"fwd+bwd with bias and db: {steps} steps")
    m, st = _timed(lambda: fldce.fldce_fwd_bwd_ex(h, W, tgt, pm, b, want_db=True, workspace=ws,
                                                  **kw), steps, warm)
    tf = 6.0 * rows_mult * H * V / (m * 1e-3) / 1e12
    out["with_bias_db"] = {"ms_per_step": round(m, 4), "tokens_per_s": round(N / (m * 1e-3), 1),
                           "tflops": round(tf, 2), "pct_peak": round(100.0 * tf / peak, 2),
                           "overhead_vs_plain": round(m / ms_plain - 1.0, 4),
                           "stage_ms_per_step": st}
    del ws
    torch.cuda.empty_cache()
    return out


def shard_bench(args, w) -> int:
    """One GPU's share of the vocabulary-split LM head (the shard workload:
    N=32768, H=5120, shard k=3 of 8, 18992 vocabulary rows): one step =
    fldce_shard_partials (softmax partials of the shard, logits never stored)
    + fldce_shard_bwd (dH_partial, dW_local given the rows' lse).  The
    exchange of partials between GPUs is not part of a one-GPU step; the lse
    passed to the backward is the shard's own (timing does not depend on its
    values)."""
    import numpy as np
    import torch
    from lm_head_linear_bf16_amd import fldce, synth
    N, H, Vl, v0 = w.N, w.H, w.V_local, w.vocab_start
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: N={N} H={H} V_local={Vl} (shard {w.shard_k} of {w.shards}); inputs")
    target, p_mask = synth.targets(w)

    def dev_t(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    h, W = dev_t(synth.hidden(w)), dev_t(synth.weight(w, shard=w.shard_k))
    tgt, pm = torch.from_numpy(target).to(dev), torch.from_numpy(p_mask).to(dev)
    dt = torch.bfloat16
    ws_p = torch.empty(fldce.fldce_shard_partials_workspace_size(N, H, Vl, dt), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(fldce.fldce_shard_bwd_workspace_size(N, H, Vl, dt), dtype=torch.uint8,
                       device=dev)
    r = fldce.fldce_shard_partials(h, W, tgt, v0, logit_scale=w.logit_scale, workspace=ws_p)
    lse = (r["row_max"] + torch.log(r["row_sumexp"])).nan_to_num(0.0, 0.0, 0.0).contiguous()
    kw = dict(label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
              reduction=w.reduction, total=w.total)

    def partials():
        return fldce.fldce_shard_partials(h, W, tgt, v0, logit_scale=w.logit_scale,
                                          sumlogit=w.label_smoothing > 0, workspace=ws_p)

    def bwd():
        return fldce.fldce_shard_bwd(h, W, tgt, pm, lse, v0, w.V, workspace=ws_b, **kw)

    log(f"timing {args.steps} steps after {args.warmup} warmup")
    mp, sp = _timed(partials, args.steps, args.warmup)
    mb, sb = _timed(bwd, args.steps, args.warmup)
    ms = mp + mb
    n_valid = int(np.count_nonzero(target != synth.IGNORE_INDEX))
    peak = PEAK_BF16_TFLOPS
    gemm = 2.0 * n_valid * H * Vl              # one GEMM over the shard, valid rows
    # dominant kernel: the GEMM stage with the largest time in either call
    # (ms per step, flops per launch)
    cands = {"partials_logits": (sp.get("logits_gemm", 0.0), gemm),
             "bwd_logits": (sb.get("logits_gemm", 0.0), gemm),
             "bwd_gemms": (sb.get("bwd_gemms", 0.0), 2 * gemm),
             "dH_gemm": (sb.get("dH_gemm", 0.0), gemm), "dW_gemm": (sb.get("dW_gemm", 0.0), gemm)}
    dom = max(cands, key=lambda k: cands[k][0])
    dom_ms, dom_flops = cands[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    result = {
        "metric": "fused LM-head CE fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), 1 GPU",
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"shard: B={w.B} L={w.L} (N={N}) H={H} V_local={Vl} "
                                f"(shard {w.shard_k} of {w.shards} of V={w.V}) eps={w.label_smoothing} "
                                f"s={w.logit_scale}, shard partials + shard backward"),
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "one vocabulary shard"},
        "tflops": round(4 * gemm / (ms * 1e-3) / 1e12, 2),
        "pct_peak": round(100.0 * 4 * gemm / (ms * 1e-3) / 1e12 / peak, 2),
        "rows_multiplied": n_valid,
        "partials": {"ms": round(mp, 4), "tflops": round(gemm / (mp * 1e-3) / 1e12, 2),
                     "stage_ms": sp,
                     "traffic_bytes": traffic_entry("partials_logits", "shard"),
                     "algorithmic_bytes": 2 * (N * H + Vl * H) + 16 * N},
        "backward": {"ms": round(mb, 4), "tflops": round(3 * gemm / (mb * 1e-3) / 1e12, 2),
                     "stage_ms": sb},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_entry(dom, "shard"), "avg_launch_ms": dom_ms,
                     "flops_per_launch": dom_flops},
        "env": env_info(torch),
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="token rows the float64 oracle baseline runs on (0 = the whole "
                         "workload: one full call, about 18 s on 16 cores at the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", default="1024,2048,4096,8192",
                    help="comma-separated row-chunk sizes to time as well ('' = none; headline "
                         "workload only)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "run with --calib-copy-mib into profiles/traffic.json and exit")
    ap.add_argument("--calib-mib", type=int, default=1024, help="size of that calibration copy")
    ap.add_argument("--counter-summary", nargs="+", metavar="RUN_DIR",
                    help="summarise rocprofv3 --pmc --kernel-trace runs (one directory each) "
                         "into profiles/<workload>_counters.md and exit")
    ap.add_argument("--counter-cmd", default="", help="the profiling command, for the summary")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the forward-only leg (and the bias + db leg)")
    ap.add_argument("--frozen-leg", action="store_true",
                    help="also time fwd+bwd without dW (a frozen weight: fldce_fwd_bwd_ex)")
    ap.add_argument("--vendor-leg", action="store_true",
                    help="also time torch.matmul (hipBLASLt) at the three GEMM shapes, for scale")
    ap.add_argument("--bias-leg", action="store_true",
                    help="also time fwd+bwd with the seeded bias and db (fldce_fwd_bwd_ex); off by "
                         "default so that the plain step is the only user of its logits kernel")
    args = ap.parse_args()
    if args.counter_summary:
        return counter_summary(args.counter_summary, args.workload, args.counter_cmd,
                               args.calib_mib)
    if args.traffic_summary:
        return traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                               args.calib_mib, cmd=args.counter_cmd)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(vocabulary and sequence sharding are described, not built).", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from lm_head_linear_bf16_amd import fldce, synth

    w = synth.WORKLOADS[args.workload]
    if w.shards > 1:
        return shard_bench(args, w)
    N, H, V = w.N, w.H, w.V
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: N={N} H={H} V={V} {w.dtype}; generating inputs")
    target, p_mask = synth.targets(w)
    hT, WT = synth.hidden(w), synth.weight(w)

    def dev_t(t):
        if t.bits is not None:
            return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.values).to(dev)

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    h, W = dev_t(hT), dev_t(WT)
    del hT, WT
    tgt = torch.from_numpy(target).to(dev)
    pm = torch.from_numpy(p_mask).to(dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def run_config(chunk_rows: int, steps: int, warmup: int, stages_pass: bool = True):
        """(ms per step, stage times, loss, per-step distribution).  The timed
        steps run with the library's stage events off; with stages_pass, the
        same number of steps then runs again with them on (not part of the
        timed figure) to give each stage's launch times."""
        out = dict(loss=torch.empty(1, dtype=torch.float32, device=dev),
                   dH=torch.empty_like(h), dW=torch.empty_like(W))
        nbytes = fldce.fldce_workspace_size(N, H, V, dt, chunk_rows)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        kw = dict(label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                  reduction=w.reduction, total=w.total, chunk_rows=chunk_rows,
                  workspace=ws, out=out)
        for _ in range(warmup):
            fldce.fldce_fwd_bwd(h, W, tgt, pm, **kw)
        torch.cuda.synchronize()
        # one event between consecutive steps on the library's stream (the
        # current one): per-step times without any synchronisation in the loop
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            fldce.fldce_fwd_bwd(h, W, tgt, pm, **kw)
            ev[i + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        loss = float(out["loss"].item())
        stages = {}
        if stages_pass:
            fldce.fldce_profile_begin()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fldce.fldce_fwd_bwd(h, W, tgt, pm, **kw)
            e1.record()
            torch.cuda.synchronize()
            fldce.fldce_profile_end()
            for s in range(fldce.fldce_profile_num_stages()):
                ms, n = fldce.fldce_profile_read(s)
                if n:
                    stages[fldce.fldce_profile_stage_name(s)] = dict(total_ms=ms, launches=n)
            stages["_step_ms_with_stage_events"] = e0.elapsed_time(e1) / steps
        del ws
        dist = {"median": round(float(np.median(per_step)), 4),
                "p10": round(float(np.percentile(per_step, 10)), 4),
                "p90": round(float(np.percentile(per_step, 90)), 4),
                "min": round(float(per_step.min()), 4)}
        return (t1 - t0) * 1e3 / steps, stages, loss, dist

    n_valid = int(np.count_nonzero(target != synth.IGNORE_INDEX))
    C = args.chunk_rows or fldce.fldce_default_chunk_rows(N, H, V)
    log(f"timing {args.steps} steps after {args.warmup} warmup (chunk_rows={C})")
    ms, stages, loss, dist = run_config(args.chunk_rows, args.steps, args.warmup)
    step_ms_profiled = stages.pop("_step_ms_with_stage_events")
    # bf16 multiplies only rows whose target != ignore_index (the others are
    # exactly zero); fp32 multiplies every row
    rows_mult = n_valid if w.dtype == "bf16" else N
    flops = 6.0 * rows_mult * H * V          # executed
    flops_nominal = 6.0 * N * H * V          # a dense pass over every row
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    # dominant kernel: the GEMM stage with the largest time; per step it does
    # 2 (one GEMM) or 4 (dH and dW) * rows * H * V flops over all its
    # launches (one per chunk)
    dom = max((k for k in stages if k in STAGE_FLOP_KERNELS), key=lambda k: stages[k]["total_ms"])
    d = stages[dom]
    per_launch_flops = STAGE_FLOP_KERNELS[dom] * rows_mult * H * V * args.steps / d["launches"]
    avg_ms = d["total_ms"] / d["launches"]
    achieved = per_launch_flops / (avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_entry(dom, w.name), "avg_launch_ms": round(avg_ms, 4),
                "flops_per_launch": per_launch_flops}
    stage_ms = {k: round(v["total_ms"] / args.steps, 4) for k, v in stages.items()}
    stage_ms["step_with_stage_events"] = round(step_ms_profiled, 4)
    result = {
        "metric": "fused LM-head CE fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), 1 GPU",
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": (f"{w.name}: B={w.B} L={w.L} (N={N}) H={H} V={V} "
                                f"eps={w.label_smoothing} s={w.logit_scale} reduction="
                                + ("sum/N" if w.total_is_N else "mean over non-ignored")),
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)",
                   "chunk_rows": int(C)},
        "tflops": round(tflops, 2),
        "pct_peak": round(100.0 * tflops / peak, 2),
        "rows_multiplied": rows_mult,
        "tflops_nominal_6NHV": round(flops_nominal / (ms * 1e-3) / 1e12, 2),
        "loss": loss,
        "step_ms": dist,
        "stage_ms_per_step": stage_ms,
        "roofline": roofline,
        "env": env_info(torch),
    }
    if not args.no_extras:
        result.update(extra_legs(args, w, h, W, tgt, pm, dt, rows_mult, ms, peak))
    if args.vendor_leg and w.dtype == "bf16":
        result["vendor_gemm"] = vendor_leg(w, rows_mult, peak)
    if args.sweep and w.name == "headline":
        # rows per chunk, taken over the compacted rows (page 1 chunks the rows
        # to bound the [C, V] buffer); C >= the rows with a target is one chunk
        sw = {}
        for c in [int(x) for x in args.sweep.split(",") if x]:
            log(f"sweep chunk_rows={c}")
            m, _, _, d = run_config(c, max(4, args.steps // 4), 1, stages_pass=False)
            sw[str(c)] = {"ms_per_step": round(m, 3), "step_ms_median": d["median"],
                          "chunks": -(-rows_mult // c), "vs_default": round(m / ms, 3),
                          "tflops": round(flops / (m * 1e-3) / 1e12, 1),
                          "tokens_per_s": round(N / (m * 1e-3), 1)}
        result["chunk_sweep"] = sw
    if not args.no_cpu_baseline:
        del h, W
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_rows or N, N))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
