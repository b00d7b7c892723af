#!/usr/bin/env python3
"""Benchmark of the online-softmax hot path on one MI355X.

One step runs every stage of the path once, each on its own synthetic batch
already resident in HBM:
  softmax_f32   row_softmax, 65536 x 8192 fp32 logits N(0,1) x 30, block 8
  softmax_bf16  row_softmax, 65536 x 8192 bf16 logits N(0,1) x 30, block 8
  attn_nc       attn_fwd, B4 H16 S2048 D64 bf16, non-causal, scale 1/8
  attn_causal   attn_fwd, B2 H32 S8192 D128 bf16, causal, scale 1/sqrt(128)
  decode        attn_decode_splitkv, B16 H32 Lmax 32768 D128 bf16, 64 splits
The headline value is the fp32 row softmax's HBM throughput (algorithmic
bytes: one read and one write of every logit); every stage is reported with
its own roofline fraction.  Each stage is timed with HIP events recorded on
the stream the kernels are launched on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Warm-up runs at least W steps and at least 0.5 s (--min-warmup-s) so the
clocks settle; then exactly K steps are timed.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "row-softmax HBM GB/s; attention fwd bf16 TFLOP/s (% of roofline), 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "row_softmax": ["tiled_exact_attention_amd/csrc/softmax.hip", "tiled_exact_attention_amd/csrc/common.hpp"],
    "attn_fwd": ["tiled_exact_attention_amd/csrc/attn_fwd.hip", "tiled_exact_attention_amd/csrc/merge.hip",
                 "tiled_exact_attention_amd/csrc/common.hpp"],
    "decode": ["tiled_exact_attention_amd/csrc/decode.hip", "tiled_exact_attention_amd/csrc/merge.hip",
               "tiled_exact_attention_amd/csrc/common.hpp"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when none exist or the kernel's source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


MAIN_STAGES = ("softmax_f32", "softmax_bf16", "attn_nc", "attn_causal", "decode")
EXTRA_STAGES = ("decode_fused", "softmax_long_f32", "attn_lowocc", "attn_lowocc_splitk",
                "softmax_f32_if_rise", "softmax_f32_l0_one", "softmax_f32_block1", "softmax_f32_block1_if_rise")
# rescale-policy A/B on the fp32 softmax batch: (rescale policy, block)
RESCALE_STAGES = {"softmax_f32_if_rise": (1, 8), "softmax_f32_l0_one": (2, 8), "softmax_f32_block1": (0, 1),
                  "softmax_f32_block1_if_rise": (1, 1)}

STAGE_KERNELS = {  # stage -> kernels (in launch order) that make up one launch: a substring of the kernel
    # name, or (substring, grid size in threads) where stages share a kernel
    "softmax_f32": ["row_softmax_kernel<false, 256, 32, true, 8, 256, 0>"],
    "softmax_bf16": ["row_softmax_kernel<true, 256, 32, true, 8, 256, 0>"],
    "softmax_f32_if_rise": ["row_softmax_kernel<false, 256, 32, true, 8, 256, 1>"],
    "softmax_f32_l0_one": ["row_softmax_kernel<false, 256, 32, true, 8, 256, 2>"],
    "softmax_f32_block1": ["row_softmax_kernel<false, 256, 32, true, 1, 256, 0>"],
    "softmax_f32_block1_if_rise": ["row_softmax_kernel<false, 256, 32, true, 1, 256, 1>"],
    "attn_nc": ["attn_fwd_kernel<64, 64, 16, true>"],
    "attn_causal": [("attn_fwd_kernel<128, 64, 8, true>", 2048 * 512)],
    "decode": ["decode_partial_kernel<128, 8>", "merge_kernel<true, true, true>"],
    "softmax_long_f32": ["row_softmax_stream_kernel<false, true, 8, 512, 0>"],
    "decode_fused": ["decode_fused_kernel<128, 4, true>"],
    "attn_lowocc": [("attn_fwd_kernel<128, 64, 8, true>", 32 * 512)],
    "attn_lowocc_splitk": [("attn_fwd_kernel<128, 64, 8, true>", 256 * 512), "merge_rows_kernel<false, true, true, 2>"],
}
STAGE_SOURCE = {"softmax_f32": "row_softmax", "softmax_bf16": "row_softmax", "attn_nc": "attn_fwd",
                "attn_causal": "attn_fwd", "decode": "decode", "softmax_long_f32": "row_softmax",
                "decode_fused": "decode", "attn_lowocc": "attn_fwd", "attn_lowocc_splitk": "attn_fwd",
                **{n: "row_softmax" for n in RESCALE_STAGES}}


def ingest_counters(fetch_csv: str, write_csv: str, command: str):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch of each stage, each counter scaled by
    what it reads for the plain 1 GiB device copy of --calibrate-copy, and
    write profiles/traffic.json (keyed by stage, with the hash of the
    kernel sources the counters were taken with)."""
    import csv
    from collections import defaultdict

    def load(path):
        per = defaultdict(list)
        copy = None
        for r in csv.DictReader(open(path)):
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name and int(r["Grid_Size"]) >= 65536:
                copy = v
            per[(name, int(r["Grid_Size"]))].append(v)
        return per, copy

    def match(per, part):
        sub, grid = (part, None) if isinstance(part, str) else part
        return [k for k in per if sub in k[0] and (grid is None or k[1] == grid)]

    fetch, fcopy = load(fetch_csv)
    write, wcopy = load(write_csv)
    gib_kib = float(1 << 20)
    rf, wf = gib_kib / fcopy, gib_kib / wcopy
    out = {"_calibration": {"copy_bytes": 1 << 30, "fetch_kib": fcopy, "write_kib": wcopy,
                            "read_factor": rf, "write_factor": wf, "command": command}}
    for stage, parts in STAGE_KERNELS.items():
        fk = wk = 0.0
        found = True
        for sub in parts:
            fn = match(fetch, sub)
            wn = match(write, sub)
            if not fn or not wn:
                found = False
                break
            fv, wv = fetch[fn[0]], write[wn[0]]
            fk += sum(fv) / len(fv)
            wk += sum(wv) / len(wv)
        if not found:
            continue
        out[stage] = {"source_hash": source_hash(STAGE_SOURCE[stage]), "fetch_kib": round(fk, 1),
                      "write_kib": round(wk, 1), "read_bytes": int(fk * 1024 * rf),
                      "write_bytes": int(wk * 1024 * wf), "bytes_per_launch": int(fk * 1024 * rf + wk * 1024 * wf)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="keep warming up until this much wall time has passed (at least --warmup steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle over every one of the five workloads in full (minutes of CPU work)")
    ap.add_argument("--stages",
                    default=",".join(MAIN_STAGES + EXTRA_STAGES))
    ap.add_argument("--no-box-references", action="store_true",
                    help="skip the copy, read and GEMM rates of this box (secondary fractions)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--ingest-command", default="", help="the rocprofv3 command the counter files came from")
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(*args.ingest_counters, args.ingest_command), indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows, heads and KV chunks would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tiled_exact_attention_amd as tea
    from tiled_exact_attention_amd import inputs

    tea.load_library()  # fail loudly before any work if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stages = args.stages.split(",")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    S = {}  # stage -> dict(fn, units, kind)
    t0 = time.perf_counter()
    rescale_stages = [n for n in RESCALE_STAGES if n in stages]
    if "softmax_f32" in stages or "softmax_bf16" in stages or rescale_stages:
        w = inputs.WORKLOADS["softmax_large"]
        R, C = w["rows"], w["cols"]
        for dt in ("f32", "bf16"):
            name = f"softmax_{dt}"
            if name not in stages and not (dt == "f32" and rescale_stages):
                continue
            x = inputs.logits(R, C, 30.0, 202 if dt == "f32" else 205, dt).to(dev)
            y = torch.empty_like(x)
            es = 4 if dt == "f32" else 2
            if name in stages:
                S[name] = dict(fn=(lambda x=x, y=y: tea.row_softmax(x, out=y, block=8)), units=R * C * 2 * es,
                               kind="hbm", kernel="row_softmax", wfrac=0.5, seed=202 if dt == "f32" else 205,
                               workload=f"row_softmax {R}x{C} {dt} N(0,1)x30 block 8")
            if dt == "f32":
                # the same batch under the other rescale policies (same bits,
                # different work per block) and at one logit per block
                for n in rescale_stages:
                    rs, blk = RESCALE_STAGES[n]
                    pol = ("unconditional", "conditional (only when the maximum rose)", "l started at 1")[rs]
                    S[n] = dict(fn=(lambda x=x, y=y, rs=rs, blk=blk: tea.row_softmax_variant(x, rs, out=y, block=blk)),
                                units=R * C * 8, kind="hbm", kernel="row_softmax", wfrac=0.5, seed=202,
                                workload=f"row_softmax {R}x{C} f32 N(0,1)x30 block {blk}, rescale {pol}")
            log(f"inputs {name} ready ({time.perf_counter() - t0:.1f}s)")
    if "softmax_long_f32" in stages:
        w = inputs.WORKLOADS["softmax_long"]  # rows longer than 16384: the two-read streaming path
        R, C = w["rows"], w["cols"]
        x = inputs.logits(R, C, 30.0, 206, "f32").to(dev)
        y = torch.empty_like(x)
        S["softmax_long_f32"] = dict(fn=(lambda x=x, y=y: tea.row_softmax(x, out=y, block=8)), units=R * C * 12,
                                     kind="hbm", kernel="row_softmax", wfrac=1 / 3, seed=206,
                                     workload=f"row_softmax {R}x{C} f32 N(0,1)x30 block 8, two reads + one write")
        log(f"inputs softmax_long_f32 ready ({time.perf_counter() - t0:.1f}s)")
    if "attn_nc" in stages:
        w = inputs.WORKLOADS["attn_noncausal"]
        B, H, Sq, D = w["B"], w["H"], w["S"], w["D"]
        q, k, v = (t.to(dev) for t in inputs.qkv(B, H, Sq, Sq, D, seed=301))
        o = torch.empty_like(q)
        S["attn_nc"] = dict(fn=(lambda q=q, k=k, v=v, o=o: tea.attn_fwd(q, k, v, causal=False, out=o)),
                            units=4 * B * H * Sq * Sq * D, kind="mfma", kernel="attn_fwd", seed=301,
                            workload=f"attn_fwd B{B} H{H} S{Sq} D{D} bf16 non-causal")
        log(f"inputs attn_nc ready ({time.perf_counter() - t0:.1f}s)")
    if "attn_lowocc" in stages or "attn_lowocc_splitk" in stages:
        w = inputs.WORKLOADS["attn_lowocc"]
        B, H, Sq, Sk, D, ns = w["B"], w["H"], w["Sq"], w["Sk"], w["D"], w["num_splits"]
        q, k, v = (t.to(dev) for t in inputs.qkv(B, H, Sq, Sk, D, seed=601))
        o = torch.empty_like(q)
        wl = f"attn_fwd B{B} H{H} Sq{Sq} Sk{Sk} D{D} bf16 non-causal ({(Sq + 255) // 256 * B * H} query blocks)"
        if "attn_lowocc" in stages:
            S["attn_lowocc"] = dict(fn=(lambda q=q, k=k, v=v, o=o: tea.attn_fwd(q, k, v, out=o)),
                                    units=4 * B * H * Sq * Sk * D, kind="mfma", kernel="attn_fwd", seed=601, workload=wl)
        if "attn_lowocc_splitk" in stages:
            wsk = torch.empty(tea.attn_fwd_splitk_workspace_bytes(B, H, Sq, D, ns), dtype=torch.uint8, device=dev)
            S["attn_lowocc_splitk"] = dict(
                fn=(lambda q=q, k=k, v=v, o=o, wsk=wsk, ns=ns: tea.attn_fwd_splitk(q, k, v, ns, workspace=wsk, out=o)),
                units=4 * B * H * Sq * Sk * D, kind="mfma", kernel="attn_fwd", seed=601, workload=wl + f", {ns} KV splits")
        log(f"inputs attn_lowocc ready ({time.perf_counter() - t0:.1f}s)")
    if "attn_causal" in stages:
        w = inputs.WORKLOADS["attn_causal"]
        B, H, Sq, D = w["B"], w["H"], w["S"], w["D"]
        q, k, v = (t.to(dev) for t in inputs.qkv(B, H, Sq, Sq, D, seed=401))
        o = torch.empty_like(q)
        S["attn_causal"] = dict(fn=(lambda q=q, k=k, v=v, o=o: tea.attn_fwd(q, k, v, causal=True, out=o)),
                                units=4 * B * H * D * Sq * (Sq + 1) // 2, kind="mfma", kernel="attn_fwd", seed=401,
                                workload=f"attn_fwd B{B} H{H} S{Sq} D{D} bf16 causal")
        log(f"inputs attn_causal ready ({time.perf_counter() - t0:.1f}s)")
    if "decode" in stages or "decode_fused" in stages:
        w = inputs.WORKLOADS["decode_splitkv"]
        B, H, Lmax, D, ns = w["B"], w["H"], w["Lmax"], w["D"], w["num_splits"]
        q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=501)
        qd, Kd, Vd, kvd = q.to(dev), K.to(dev), V.to(dev), kv.to(dev)
        del K, V
        ws = torch.empty(tea.attn_decode_workspace_bytes(B, H, D, ns), dtype=torch.uint8, device=dev)
        od = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        tot = int(kv.sum())
        S["decode"] = dict(fn=(lambda qd=qd, Kd=Kd, Vd=Vd, kvd=kvd, ns=ns, ws=ws, od=od:
                               tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=ns, workspace=ws,
                                                               out=od)),
                           units=tot * H * D * 2 * 2 + B * H * D * 2 * 2 + B * 4, kind="hbm", kernel="decode", seed=501,
                           wfrac=B * H * D * 2 / (tot * H * D * 2 * 2 + B * H * D * 2 * 2 + B * 4),
                           workload=f"decode B{B} H{H} Lmax{Lmax} D{D} bf16 splits{ns} sum(kv_len)={tot}")
        if "decode_fused" in stages:
            of = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
            S["decode_fused"] = dict(fn=(lambda qd=qd, Kd=Kd, Vd=Vd, kvd=kvd, ns=ns, of=of:
                                         tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=ns, out=of)),
                                     units=S["decode"]["units"], kind="hbm", kernel="decode", seed=501,
                                     wfrac=S["decode"]["wfrac"],
                                     workload=S["decode"]["workload"] + ", one launch")
        if "decode" not in stages:
            del S["decode"]
        log(f"inputs decode ready ({time.perf_counter() - t0:.1f}s)")

    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write done")
        del a, b

    stream = torch.cuda.current_stream(dev)
    # the step: one pass of the hot path's rows; the variants built beside it
    # (long rows, one-launch decode, split-K attention) are timed after the
    # steps, each in a loop of its own, and are not part of ms_per_step
    names = [n for n in MAIN_STAGES if n in S]
    extras = [n for n in EXTRA_STAGES if n in S]

    def step(events=None):
        for n in names:
            if events is not None:
                events[n][0].record(stream)
            S[n]["fn"]()
            if events is not None:
                events[n][1].record(stream)

    # Warm-up: at least W steps and at least --min-warmup-s seconds of GPU
    # work, so the engine clock has settled before the timed steps (a cold
    # MI355X runs its first ~10 ms of MFMA work measurably slower).
    nwarm = 0
    w0 = time.perf_counter()
    while nwarm < args.warmup or time.perf_counter() - w0 < args.min_warmup_s:
        step()
        torch.cuda.synchronize()
        nwarm += 1
    log(f"warmup {nwarm} steps done ({time.perf_counter() - w0:.2f}s)")

    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    log(f"timed {args.steps} steps in {w1 - w0:.3f}s")
    ms_per_step = (w1 - w0) * 1e3 / max(args.steps, 1)

    times = {n: [evs[i][n][0].elapsed_time(evs[i][n][1]) for i in range(args.steps)] for n in names}
    for n in extras:
        fn = S[n]["fn"]
        w0 = time.perf_counter()
        k = 0
        while k < args.warmup or time.perf_counter() - w0 < args.min_warmup_s / 2:
            fn()
            torch.cuda.synchronize()
            k += 1
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        times[n] = [a.elapsed_time(b) for a, b in ev]
        log(f"extra stage {n}: {k} warm-up and {args.steps} timed calls")

    box = None if (args.calibrate_copy or args.no_box_references) else box_references(dev, stream)
    if box:
        log(f"box references: copy {box['copy_GBps']:.0f} GB/s, read {box['read_GBps']:.0f} GB/s, "
            f"bf16 GEMM {box['gemm_bf16_TFLOPs']:.0f} TFLOP/s")

    paths = {}
    for n in names + extras:
        t = times[n]
        avg = float(np.mean(t))
        s = S[n]
        if s["kind"] == "hbm":
            ach = s["units"] / (avg * 1e-3) / 1e9
            peak, unit = HBM_PEAK_GBS, "GB/s"
        else:
            ach = s["units"] / (avg * 1e-3) / 1e12
            peak, unit = BF16_PEAK_TFLOPS, "TFLOP/s"
        paths[n] = {
            "workload": s["workload"], "seed": s["seed"], "in_step": n in names, "avg_ms": round(avg, 5),
            "min_ms": round(float(np.min(t)), 5),
            "median_ms": round(float(np.median(t)), 5),
            "roofline": {"bound": s["kind"], "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4), "traffic": measured_traffic(s["kernel"], n),
                         "algorithmic_units_per_launch": s["units"]},
        }
        if box:
            if s["kind"] == "hbm":
                # what this box's copy and read kernels would take for the
                # same bytes: the written bytes and as many read ones as a
                # copy, the remaining reads as a pure read
                f = s["wfrac"]
                t_box = 2 * f / box["copy_GBps"] + (1 - 2 * f) / box["read_GBps"]
                paths[n]["frac_of_box"] = round(ach * t_box, 4)
            else:
                paths[n]["frac_of_box"] = round(ach / box["gemm_bf16_TFLOPs"], 4)

    # the headline: the fp32 row softmax when it ran, else the first stage run
    head = "softmax_f32" if "softmax_f32" in paths else (names + extras)[0]
    hp = paths[head]
    out = {
        "metric": METRIC,
        "value": hp["roofline"]["achieved"],
        "unit": hp["roofline"]["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": nwarm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        # inputs: numpy default_rng streams keyed by each stage's seed
        # (tiled_exact_attention_amd.inputs), bf16 rounded by torch
        "inputs": {"numpy": np.__version__, "torch": torch.__version__},
        "config": {"workload": hp["workload"], "stages": names, "extra_stages": extras},
        "roofline": hp["roofline"],
        "paths": paths,
    }
    if box:
        out["box_references"] = box
    if "attn_causal" in paths:
        out["attention_tflops"] = paths["attn_causal"]["roofline"]["achieved"]

    if not args.no_cpu_baseline and "softmax_f32" in S:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    if args.cpu_full:
        out["cpu_full"] = cpu_full()
    print(json.dumps(out), flush=True)


def box_references(dev, stream):
    """Rates this box reaches with plain library kernels, for secondary
    fractions: a 1 GiB device copy (bytes read + written), a 1 GiB fp32 sum
    (bytes read) and an 8192^3 bf16 GEMM (torch.mm, contiguous operands)."""
    import numpy as np
    import torch

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e-3

    x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    x.fill_(1.0)
    y = torch.empty_like(x)
    t_copy = timed(lambda: y.copy_(x), 10)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    t_read = timed(lambda: torch.sum(x, 0, out=acc), 10)
    del x, y
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    t_gemm = timed(lambda: torch.mm(a, b, out=c), 10)
    del a, b, c
    return {"copy_GBps": round(2 * (1 << 30) / t_copy / 1e9, 1), "read_GBps": round((1 << 30) / t_read / 1e9, 1),
            "gemm_bf16_TFLOPs": round(2 * n ** 3 / t_gemm / 1e12, 1),
            "how": "device copy of 1 GiB (read + write bytes), fp32 sum of 1 GiB (read bytes), torch.mm bf16 "
                   "8192^3; medians of 10; frac_of_box = achieved / the rate these give for the same bytes or flops"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, budget_s: float):
    """Run fn() repeatedly until about budget_s has passed; (calls, seconds)."""
    n, t = 0, 0.0
    while n == 0 or t < budget_s:
        s = time.perf_counter()
        fn()
        t += time.perf_counter() - s
        n += 1
    return n, t


def cpu_baseline(budget_s: float):
    """The fp64 CPU oracle, as it stands, timed on the host cores on bounded
    samples of the same seeded workloads, each scaled to its stage's unit:
      value   the headline row softmax 65536 x 8192 fp32 (GB/s of logits read
              and written), the first rows of the same batch;
      paths   the 4096 x 1024 softmax on one thread; attention B4 H16 S2048
              D64 and causal B2 H32 S8192 D128 on every 64th / 256th query
              row (TFLOP/s of the rows' algorithmic flop); split-KV decode on
              the 32 heads of two sequences (GB/s of their K and V)."""
    import numpy as np

    import oracle
    from tiled_exact_attention_amd import inputs

    threads = oracle.num_threads()
    out = {"unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "host_cpu_count": os.cpu_count()}

    # headline: the fp32 row softmax, grown to about budget_s / 4 per pass
    C = inputs.WORKLOADS["softmax_large"]["cols"]
    x = inputs.logits(65536, C, 30.0, 202, "f32").numpy()
    rows = 256
    while True:
        s = time.perf_counter()
        oracle.softmax_rows(x[:rows])
        t = time.perf_counter() - s
        if t >= budget_s / 4 or rows >= 65536:
            break
        rows = min(65536, int(rows * max(2.0, budget_s / 4 / max(t, 1e-3))))
    reps = 1
    while t < 0.8 * budget_s:
        s = time.perf_counter()
        oracle.softmax_rows(x[:rows])
        t += time.perf_counter() - s
        reps += 1
    del x
    out["value"] = round(rows * C * 8 * reps / t / 1e9, 4)
    out["sample"] = (f"first {rows} of 65536 rows x {C} fp32 logits (same seeded batch), {reps} pass(es), "
                     f"fp64 two-pass oracle with OpenMP, {t:.2f}s")
    paths = {}

    # the small softmax configuration on one thread
    w = inputs.WORKLOADS["softmax_small"]
    xs = inputs.logits(w["rows"], w["cols"], 1.0, 101, "f32").numpy()
    prev = oracle.set_num_threads(1)
    try:
        n, t = _timed(lambda: oracle.softmax_rows(xs), 2.0)
    finally:
        oracle.set_num_threads(prev)
    paths["softmax_small_1thread"] = {"value": round(xs.size * 8 * n / t / 1e9, 4), "unit": "GB/s", "cores": 1,
                                      "sample": f"all {w['rows']} x {w['cols']} fp32 logits x1 (seed 101), {n} pass(es), "
                                                f"{t:.2f}s"}

    # attention: sampled query rows of the two workloads
    for name, key, seed, step in (("attn_nc", "attn_noncausal", 301, 64), ("attn_causal", "attn_causal", 401, 256)):
        w = inputs.WORKLOADS[key]
        B, H, S, D, causal = w["B"], w["H"], w["S"], w["D"], w["causal"]
        q, k, v = (a.float().numpy() for a in inputs.qkv(B, H, S, S, D, seed=seed))
        flat = np.arange(0, B * H * S, step, dtype=np.int64)
        keys = (flat % S + 1) if causal else np.full(flat.shape, S)
        flop = int(4 * D * keys.sum())
        n, t = _timed(lambda: oracle.attention(q, k, v, 1.0 / np.sqrt(D), causal, rows=flat), 2.0)
        paths[name] = {"value": round(flop * n / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
                       "sample": f"every {step}th of {B * H * S} query rows ({len(flat)} rows, {keys.sum()} visible "
                                 f"keys) of the seeded workload, {n} pass(es), {t:.2f}s"}
        del q, k, v

    # split-KV decode: every head of the first two sequences
    w = inputs.WORKLOADS["decode_splitkv"]
    B, H, Lmax, D = w["B"], w["H"], w["Lmax"], w["D"]
    kv_len = inputs.kv_lengths(B, Lmax, 501)
    qd = inputs.decode_q(B, H, D, 501)
    sel = [0, 1]
    data = []
    for b in sel:
        L = int(kv_len[b])
        kk = np.stack([inputs.decode_kv_pair(b, h, L, D, 501)[0] for h in range(H)])[None]
        vv = np.stack([inputs.decode_kv_pair(b, h, L, D, 501)[1] for h in range(H)])[None]
        data.append((qd[b][None, :, None, :], kk, vv))
    nbytes = sum(2 * kk.size * 2 for _, kk, _ in data)  # K and V as bf16
    n, t = _timed(lambda: [oracle.attention(qq, kk, vv, 1.0 / np.sqrt(D), False) for qq, kk, vv in data], 2.0)
    paths["decode"] = {"value": round(nbytes * n / t / 1e9, 4), "unit": "GB/s", "cores": threads,
                       "sample": f"all {H} heads of sequences {sel} (kv_len {[int(kv_len[b]) for b in sel]}) of the "
                                 f"seeded workload, {n} pass(es), {t:.2f}s"}
    out["paths"] = paths
    return out


def cpu_full():
    """The fp64 oracle over each of the five workloads in full, once, on all
    host threads: every row of the softmax batches (4096 x 1024 at x1 and
    x1000 with the 64-logit vectors; 65536 x 8192 fp32 and bf16 at x1, x30
    and x1000), every query row of both attention workloads, every (b, h) of
    the decode.  Seconds per workload and the rate in each stage's unit."""
    import numpy as np

    import oracle
    from tiled_exact_attention_amd import inputs

    res = {"cores": oracle.num_threads(), "cpu_model": cpu_model()}

    def clock(fn):
        s = time.perf_counter()
        fn()
        return time.perf_counter() - s

    w = inputs.WORKLOADS["softmax_small"]
    t = 0.0
    for scale, seed in ((1.0, 101), (1000.0, 102)):
        x = inputs.logits(w["rows"], w["cols"], scale, seed, "f32").numpy()
        t += clock(lambda: oracle.softmax_rows(x))
    for scale, seed in ((1.0, 103), (1000.0, 104)):
        v = inputs.vector64(scale, seed).astype(np.float32)[None]
        t += clock(lambda: oracle.softmax_rows(v))
    res["softmax_small"] = {"seconds": round(t, 3), "GB/s": round((2 * w["rows"] * w["cols"] + 2 * 64) * 8 / t / 1e9, 3)}
    log(f"cpu_full softmax_small {t:.2f}s")
    w = inputs.WORKLOADS["softmax_large"]
    t = 0.0
    for dt, seeds in (("f32", (201, 202, 203)), ("bf16", (204, 205, 206))):
        for scale, seed in zip((1.0, 30.0, 1000.0), seeds):
            x = inputs.logits(w["rows"], w["cols"], scale, seed, dt).float().numpy()
            for r0 in range(0, w["rows"], 8192):  # bounded memory: 8192 rows of fp64 output at a time
                t += clock(lambda: oracle.softmax_rows(x[r0:r0 + 8192]))
            del x
            log(f"cpu_full softmax_large {dt} x{scale} done ({t:.2f}s of oracle so far)")
    res["softmax_large"] = {"seconds": round(t, 3), "rows": 6 * w["rows"],
                            "GB/s (fp32-equivalent bytes)": round(6 * w["rows"] * w["cols"] * 8 / t / 1e9, 3)}
    for name, key, seed in (("attn_nc", "attn_noncausal", 301), ("attn_causal", "attn_causal", 401)):
        w = inputs.WORKLOADS[key]
        B, H, S, D, causal = w["B"], w["H"], w["S"], w["D"], w["causal"]
        q, k, v = (a.float().numpy() for a in inputs.qkv(B, H, S, S, D, seed=seed))
        t = 0.0
        step = 8192
        for r0 in range(0, B * H * S, step):
            rows = np.arange(r0, min(B * H * S, r0 + step), dtype=np.int64)
            t += clock(lambda: oracle.attention(q, k, v, 1.0 / np.sqrt(D), causal, rows=rows))
            if (r0 // step) % 8 == 7:
                log(f"cpu_full {name}: {r0 + step} of {B * H * S} rows ({t:.1f}s)")
        flop = 4 * B * H * D * (S * (S + 1) // 2 if causal else S * S)
        res[name] = {"seconds": round(t, 3), "TFLOP/s": round(flop / t / 1e12, 6)}
        log(f"cpu_full {name} {t:.2f}s")
        del q, k, v
    w = inputs.WORKLOADS["decode_splitkv"]
    B, H, Lmax, D = w["B"], w["H"], w["Lmax"], w["D"]
    kv_len = inputs.kv_lengths(B, Lmax, 501)
    qd = inputs.decode_q(B, H, D, 501)
    t = 0.0
    for b in range(B):
        L = int(kv_len[b])
        pairs = [inputs.decode_kv_pair(b, h, L, D, 501) for h in range(H)]
        kk = np.stack([p[0] for p in pairs])[None]
        vv = np.stack([p[1] for p in pairs])[None]
        t += clock(lambda: oracle.attention(qd[b][None, :, None, :], kk, vv, 1.0 / np.sqrt(D), False))
    res["decode"] = {"seconds": round(t, 3), "GB/s": round(int(kv_len.sum()) * H * D * 2 * 2 / t / 1e9, 3)}
    log(f"cpu_full decode {t:.2f}s")
    return res


if __name__ == "__main__":
    main()
