#!/usr/bin/env python3
"""Benchmark of the fused W4A4 + low-rank linear layer (SVDQuant) on one MI355X.

One step = one pass of the whole hot path over one batch: kernel 1 (smoothing,
4-bit quantization, low-rank down projection) then kernel 2 (4-bit GEMM with
per-group rescale and the low-rank up projection), through svdq_linear_forward,
with X already resident in HBM.  The weights are packed once beforehand by the
library's host-side svdq_pack_weights (offline, untimed).

Workload (default): the FLUX.1 QKV projection, X bf16 [4608 x 3072] (4096 image +
512 text tokens), W [3072 x 9216], rank 32, INT4 group 64 with fp16 scales, fp32
output; synthetic seeded data of that shape.

Prints one JSON line.  `value` is layer TOPS = (2 M N K + 2 M r (K + N)) / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused W4A4+low-rank linear TOPS at FLUX shapes; % of MFMA peak (1 GPU)"
PEAK_MFMA_TOPS = 5000.0  # MI355X dense INT8 / FP8 MFMA, 5.0 POP/s
PEAK_MFMA_FP4_TOPS = 10100.0  # dense MXFP4 / FP6
PEAK_HBM_GBS = 8000.0
K2_SOURCES = ["bit_diffusion_model_amd/csrc/k2_gemm_w4a4.hip", "bit_diffusion_model_amd/csrc/common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k2_gemm_int4_flux_qkv_traffic.json")

WORKLOADS = {"C1": "FLUX.1 QKV projection", "C2a": "FLUX.1 MLP fc1", "C2b": "FLUX.1 MLP fc2",
             "C3": "FLUX.1 QKV projection, MXFP4", "C4": "FLUX.1 QKV projection at batch 2 + rank-16 LoRA",
             "C0": "tiny layer"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry():
    """Measured HBM bytes per kernel-2 launch from the committed rocprofv3 counter
    summary, or None when the kernel source changed since those counters were taken."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("k2_source_hash") != source_hash(K2_SOURCES):
        return None
    return d.get("bytes_per_launch")


CALIB_BYTES = 512 << 20


def _pmc_means(path):
    """Mean counter value per kernel-name prefix from a rocprofv3 counter CSV."""
    import csv
    import collections

    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        # kernel 2 of the timed forward: the INT4 streamed kernel on the MMA activation
        # form (the fixup launch is counted with it)
        if "k2_stream<0>" in name or "k2_fixup" in name:
            key = "k2" if "k2_stream" in name else "fixup"
        elif "copyBuffer" in name or "copy" in name.lower():
            key = "copy"
        else:
            key = None
        if key:
            acc[key].append(float(r["Counter_Value"]))
    # the calibration copy is the largest copy dispatch (uploads may also use copy kernels)
    return {k: ((max(v) if k == "copy" else sum(v) / len(v)), len(v)) for k, v in acc.items()}


def write_traffic(fetch_csv, write_csv):
    """Kernel 2's HBM traffic per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    of kernel 2, each divided by the same counter's reading per byte for a plain copy of
    CALIB_BYTES (read and written once each)."""
    f = _pmc_means(fetch_csv)
    w = _pmc_means(write_csv)
    ffac = f["copy"][0] * 1024.0 / CALIB_BYTES
    wfac = w["copy"][0] * 1024.0 / CALIB_BYTES
    # the fixup launch runs once per kernel-2 launch
    fetch_b = (f["k2"][0] + f.get("fixup", (0.0, 0))[0]) * 1024.0 / ffac
    write_b = (w["k2"][0] + w.get("fixup", (0.0, 0))[0]) * 1024.0 / wfac
    d = {"kernel": "k2_stream<INT4> + k2_fixup", "workload": "FLUX.1 QKV projection M=4608 K=3072 N=9216 r=32, fp32 Y",
         "k2_source_hash": source_hash(K2_SOURCES), "fetch_kib_raw": f["k2"][0], "write_kib_raw": w["k2"][0],
         "copy_fetch_factor": ffac, "copy_write_factor": wfac, "fetch_bytes": fetch_b, "write_bytes": write_b,
         "bytes_per_launch": fetch_b + write_b, "dispatches": f["k2"][1],
         "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                    "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-compare --calib-copy"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d))


def cpu_baseline(wl_name, rows):
    """The oracle forward (unchanged, numpy fp64 / exact integers) on a bounded sample:
    `rows` tokens of the workload against all output columns.  Pack artifacts are
    seeded synthetic arrays of the right shapes (timing does not depend on values)."""
    from bit_diffusion_model_amd.workloads import make
    from oracle import forward as oforward

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    wl = make(wl_name)
    rng = np.random.default_rng(0)
    K, N, r = wl.K, wl.N, wl.total_rank
    G = wl.group
    packed = dict(
        fmt=wl.fmt, inv_s32=rng.uniform(0.2, 2, K).astype(np.float32),
        L1b=rng.standard_normal((K, r)), L2b=rng.standard_normal((r, N)),
        codesW=(rng.integers(-7, 8, (N, K)).astype(np.int8) if wl.fmt == "int4"
                else rng.integers(0, 16, (N, K)).astype(np.uint8)),
        sW=(rng.uniform(0.01, 1, (K // G, N)).astype(np.float16).view(np.uint16) if wl.fmt == "int4"
            else rng.integers(120, 134, (K // G, N)).astype(np.uint8)),
    )
    X = wl.X[:rows]
    t0 = time.perf_counter()
    oforward.forward(X, packed)
    t = time.perf_counter() - t0
    ops = 2.0 * rows * N * K + 2.0 * rows * r * (K + N)
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle forward on {rows} of {wl.M} tokens x all {N} outputs of the {WORKLOADS[wl_name]} "
                      f"layer ({t:.1f} s); host {os.cpu_count()} logical CPUs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~60 ms of warm-up (the clocks settle within a few tens of ms) and of
    # timed work at C1
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="C1", choices=list(WORKLOADS))
    ap.add_argument("--ydtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--cpu-rows", type=int, default=4608)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the rank-0 and unfused comparison forwards (counter runs: only the "
                         "timed layer's kernels are dispatched)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain device copy of 512 MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="compute kernel 2's HBM bytes per launch from two rocprofv3 --pmc CSVs "
                         "(FETCH_SIZE, WRITE_SIZE) of runs made with --calib-copy, write the "
                         "summary JSON, and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU: the layer shards along tokens with no "
                                   "exchange step, and only the one-GPU share is implemented and timed; "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import torch
    from bit_diffusion_model_amd import svdq
    from bit_diffusion_model_amd.workloads import make

    svdq.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = "cuda:0"
    wl = make(args.workload)
    M, K, N = wl.M, wl.K, wl.N
    fmt = svdq.FMT[wl.fmt]
    log(f"[bench] workload {args.workload} M={M} K={K} N={N} r={wl.rank} fmt={wl.fmt}; packing on host")
    t0 = time.perf_counter()
    hp = svdq.pack_weights(wl.W, svdq.act_absmax(wl.calib), wl.alpha, wl.rank, fmt)
    if wl.lora_A is not None:
        hp = svdq.concat_lora(hp, wl.lora_A, wl.lora_B)
    log(f"[bench] pack {time.perf_counter() - t0:.1f} s (offline, untimed)")
    lay = svdq.PackedLinear.from_host_pack(hp, dev)
    lay0 = svdq.PackedLinear(K, N, 0, fmt, hp.inv_s, hp.L1t[:0], hp.L2[:0], hp.qW, hp.sW, dev)
    r = hp.rank
    X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.bfloat16)
    ydt = svdq.F32 if args.ydtype == "f32" else svdq.BF16
    Y = torch.empty((M, N), dtype=torch.float32 if ydt == svdq.F32 else torch.bfloat16, device=dev)
    ws = lay.workspace(M)
    ws0 = lay0.workspace(M)

    def step():
        lay.forward(X, ydt, Y, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done; timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
    tops = ops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.4f} ms/step (wall {wall / args.steps * 1e3:.4f}), {tops:.1f} TOPS")

    # per-kernel durations, launched exactly as inside svdq_linear_forward (activation
    # side in MMA form), on the same (torch current) stream the events are recorded on
    qX, sX, la = lay.alloc_act(M, svdq.ACT_MMA)
    gws = lay.gemm_workspace(M, svdq.ACT_MMA)
    nrep = max(args.steps, 10)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3 * nrep)]
    for i in range(nrep):
        e[3 * i].record()
        lay.quantize_act(X, (qX, sX, la), form=svdq.ACT_MMA)
        e[3 * i + 1].record()
        lay.gemm(qX, sX, la, ydt, Y, form=svdq.ACT_MMA, workspace=gws)
        e[3 * i + 2].record()
    torch.cuda.synchronize()
    t_k1 = float(np.mean([e[3 * i].elapsed_time(e[3 * i + 1]) for i in range(nrep)])) * 1e-3
    t_k2 = float(np.mean([e[3 * i + 1].elapsed_time(e[3 * i + 2]) for i in range(nrep)])) * 1e-3
    # low-rank overhead: the layer against a rank-0 layer with the same codes, and against
    # the unfused baseline (the low-rank branch as kernels of its own), timed in alternating
    # blocks of 20 forwards (medians of 5), so all three see the same clocks
    fr, f0, fu = [], [], []
    for _ in range(0 if args.no_compare else 5):
        for lyr, wsp, fused, out in ((lay, ws, True, fr), (lay0, ws0, True, f0), (lay, ws, False, fu)):
            lyr.forward(X, ydt, Y, wsp, fused=fused)
            ev0.record()
            for _ in range(20):
                lyr.forward(X, ydt, Y, wsp, fused=fused)
            ev1.record()
            torch.cuda.synchronize()
            out.append(ev0.elapsed_time(ev1) / 20)
    med = lambda v: float(np.median(v)) if v else float("nan")
    rnd = lambda x, d: None if x != x else round(x, d)  # NaN (not measured) -> null
    ms_r, ms0, ms_u = med(fr), med(f0), med(fu)

    G = lay.group
    k2_ops = float(M) * N * (2.0 * K + 2.0 * r)
    # kernel 1's HBM bytes in MMA form: X (bf16), codes (INT4 FP6 operand words, 64 bytes
    # per group / MXFP4 nibbles), scales (INT4 fp16 / E8M0 bytes), lora_act (R16 x 4
    # bytes); the factor rows are re-read from L2 and not counted
    if fmt == svdq.INT4_G64:
        k1_bytes = float(M) * (2 * K + K + (K // G) * 2 + 4 * svdq.r16(r))
    else:
        k1_bytes = float(M) * (2 * K + K // 2 + (K // G) + 4 * svdq.r16(r))
    peak = PEAK_MFMA_TOPS if fmt == svdq.INT4_G64 else PEAK_MFMA_FP4_TOPS
    k2_tops = k2_ops / t_k2 / 1e12
    traffic = traffic_entry() if args.workload == "C1" and ydt == svdq.F32 else None
    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4" if fmt == svdq.INT4_G64 else "fp4-e2m1", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "M": M, "K": K, "N": N, "rank": r,
                   "format": "INT4 g64 fp16 scales" if fmt == svdq.INT4_G64 else "MXFP4 g32 E8M0 scales",
                   "output": args.ydtype, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(k2_tops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(k2_tops / peak, 4), "traffic": traffic},
        "kernels": {"k1_us": round(t_k1 * 1e6, 2), "k2_us": round(t_k2 * 1e6, 2),
                    "k1_GBps": round(k1_bytes / t_k1 / 1e9, 1), "k1_hbm_frac": round(k1_bytes / t_k1 / 1e9 / PEAK_HBM_GBS, 4),
                    "k2_TOPS": round(k2_tops, 2), "rank0_ms": rnd(ms0, 5),
                    "fwd_ms_paired": rnd(ms_r, 5), "lowrank_overhead": rnd(ms_r / ms0 - 1.0, 4),
                    "unfused_ms": rnd(ms_u, 5), "unfused_lowrank_overhead": rnd(ms_u / ms0 - 1.0, 4)},
    }
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} tokens")
        out["cpu_baseline"] = cpu_baseline(args.workload, min(args.cpu_rows, M))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
