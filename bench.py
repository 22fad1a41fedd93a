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
             "C0": "tiny layer", "C1nv": "FLUX.1 QKV projection, NVFP4-style group-16 two-level scales"}
PEAK_BF16_TOPS = 2500.0  # dense fp16 / bf16 MFMA, what the NVFP4 kernel 2 runs on


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


def _kernel_key(name, fmt=0):
    """Which launch of the timed forward a rocprofv3 kernel name is: kernel 1, kernel 2
    (the streamed kernel of format fmt on the MMA activation form: 0 INT4, 1 MXFP4),
    kernel 2's K-split fixup, or a device copy (the calibration copy is the largest of
    those)."""
    if "k1_quant_lora_down" in name:
        return "k1"
    if f"k2_stream<{fmt}" in name:
        return "k2"
    if "k2_fixup" in name:
        return "fixup"
    if "k2_" in name or "k3_" in name:
        return None
    return "copy" if "copy" in name.lower() else None


def _pmc_table(path, fmt=0):
    """{kernel key: {counter: (mean over dispatches, dispatches)}} from a rocprofv3
    counter CSV; for the copy key the largest dispatch."""
    import csv
    import collections

    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        key = _kernel_key(r["Kernel_Name"], fmt)
        if key:
            acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: ((max(v) if k == "copy" else sum(v) / len(v)), len(v)) for c, v in cs.items()}
            for k, cs in acc.items()}


PMC_COMMAND = ("rocprofv3 --pmc {counters} --output-format csv -d <dir> -o <name> -- python bench.py --steps 3 "
               "--warmup 1 --warm-seconds 0 --no-cpu-baseline --no-compare --no-others --calib-copy")


def write_traffic(fetch_csv, write_csv):
    """HBM traffic per launch of kernel 1 and of kernel 2 (with its fixup): FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each divided by the same counter's reading per byte
    for a plain copy of CALIB_BYTES (read and written once each)."""
    f = _pmc_table(fetch_csv)
    w = _pmc_table(write_csv)
    ffac = f["copy"]["FETCH_SIZE"][0] * 1024.0 / CALIB_BYTES
    wfac = w["copy"]["WRITE_SIZE"][0] * 1024.0 / CALIB_BYTES
    val = lambda t, k, c: t.get(k, {}).get(c, (0.0, 0))[0]
    # the fixup launch runs once per kernel-2 launch
    fetch_b = (val(f, "k2", "FETCH_SIZE") + val(f, "fixup", "FETCH_SIZE")) * 1024.0 / ffac
    write_b = (val(w, "k2", "WRITE_SIZE") + val(w, "fixup", "WRITE_SIZE")) * 1024.0 / wfac
    k1_f = val(f, "k1", "FETCH_SIZE") * 1024.0 / ffac
    k1_w = val(w, "k1", "WRITE_SIZE") * 1024.0 / wfac
    d = {"kernel": "k2_stream<INT4> + k2_fixup", "workload": "FLUX.1 QKV projection M=4608 K=3072 N=9216 r=32, fp32 Y",
         "k2_source_hash": source_hash(K2_SOURCES), "fetch_kib_raw": val(f, "k2", "FETCH_SIZE"),
         "write_kib_raw": val(w, "k2", "WRITE_SIZE"), "copy_fetch_factor": ffac, "copy_write_factor": wfac,
         "fetch_bytes": fetch_b, "write_bytes": write_b, "bytes_per_launch": fetch_b + write_b,
         "dispatches": f["k2"]["FETCH_SIZE"][1],
         "k1": {"kernel": "k1_quant_lora_down<INT4, MMA form>", "fetch_bytes": k1_f, "write_bytes": k1_w,
                "bytes_per_launch": k1_f + k1_w,
                "algorithmic_bytes": k1_algorithmic_bytes(4608, 3072, 64, 32, True)},
         "command": PMC_COMMAND.format(counters="FETCH_SIZE") + "; the same with --pmc WRITE_SIZE; then "
                    "python bench.py --write-traffic <fetch csv> <write csv>"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d))


COUNTERS_FILE = os.path.join(ROOT, "profiles", "k2_gemm_int4_flux_qkv_counters.json")
COUNTERS_FILE_MX = os.path.join(ROOT, "profiles", "k2_gemm_mxfp4_flux_qkv_counters.json")
N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4


def write_counters(a_csv, b_csv, workload="C1"):
    """Utilisation of kernels 1 and 2 from two rocprofv3 --pmc passes.  GRBM_GUI_ACTIVE is
    summed over the 8 XCDs, so one XCD's active cycles are a eighth of it; the SQ busy
    counters are summed over all 1024 SIMDs (SQ_ACTIVE_INST_VALU in units of 4 cycles,
    one wave64 VALU issue), so each fraction below is per SIMD-cycle of the launch."""
    mx = workload == "C3"
    fmt = 1 if mx else 0
    a, b = _pmc_table(a_csv, fmt), _pmc_table(b_csv, fmt)
    wflag = " --workload C3" if mx else ""
    out = {"workload": "FLUX.1 QKV projection M=4608 K=3072 N=9216 r=32, "
                       + ("MXFP4 g32" if mx else "INT4 g64") + ", fp32 Y",
           "k2_source_hash": source_hash(K2_SOURCES),
           "commands": [PMC_COMMAND.format(counters=" ".join(sorted(a["k2"]))) + wflag,
                        PMC_COMMAND.format(counters=" ".join(sorted(b["k2"]))) + wflag,
                        "python bench.py --write-counters <pass A csv> <pass B csv>" + wflag],
           "kernels": {}}
    for key in ("k1", "k2"):
        raw = {c: v[0] for c, v in a.get(key, {}).items()}
        raw.update({c: v[0] for c, v in b.get(key, {}).items() if c != "GRBM_GUI_ACTIVE"})
        cyc = raw["GRBM_GUI_ACTIVE"] / N_XCD
        simd_cyc = cyc * N_CU * SIMD_PER_CU
        g = lambda c: raw.get(c, float("nan"))
        hits, miss = g("TCC_HIT_sum"), g("TCC_MISS_sum")
        out["kernels"][key] = {
            "raw_mean_per_dispatch": raw,
            "active_cycles_per_xcd": cyc,
            "mfma_busy_frac": g("SQ_VALU_MFMA_BUSY_CYCLES") / simd_cyc,
            "valu_busy_frac": 4.0 * g("SQ_ACTIVE_INST_VALU") / simd_cyc,
            "valu_mfma_coexec_frac": g("SQ_VALU_MFMA_COEXEC_CYCLES") / simd_cyc,
            "valu_insts_per_mfma": g("SQ_INSTS_VALU") / max(g("SQ_INSTS_MFMA"), 1.0),
            "lds_bank_conflict_cycles_per_lds_inst": g("SQ_LDS_BANK_CONFLICT") / max(g("SQ_INSTS_LDS"), 1.0),
            "l2_hit_frac": hits / (hits + miss) if hits + miss > 0 else None}
    with open(COUNTERS_FILE_MX if mx else COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


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
    # the same on one BLAS thread, on a sixteenth of the rows
    rows1 = max(rows // 16, 1)
    t1 = None
    try:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oforward.forward(wl.X[:rows1], packed)
            t1 = time.perf_counter() - t0
    except Exception:  # pragma: no cover
        pass
    ops1 = 2.0 * rows1 * N * K + 2.0 * rows1 * r * (K + N)
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle forward on {rows} of {wl.M} tokens x all {N} outputs of the {WORKLOADS[wl_name]} "
                      f"layer ({t:.1f} s); host {os.cpu_count()} logical CPUs ({model})",
            "single_thread": (None if t1 is None else
                              {"value": ops1 / t1 / 1e12, "unit": "TOPS", "cores": 1,
                               "sample": f"oracle forward on {rows1} tokens x all {N} outputs, one BLAS thread "
                                         f"({t1:.1f} s)"})}


PEAK_INT8_TOPS = PEAK_MFMA_TOPS


def k1_algorithmic_bytes(M, K, G, r, int4):
    """Kernel 1's algorithmic HBM bytes: per token 2K (bf16 X) + K/2 (4-bit codes) +
    (K/G) x (2-byte fp16 / 1-byte E8M0 scale) + 4r (fp32 X_hat L1).  The factor rows are
    re-read from cache and not counted; the wider operand form the forward writes is not
    counted either."""
    return float(M) * (2 * K + K // 2 + (K // G) * (2 if int4 else 1) + 4 * r)


def percentiles_us(ms_list):
    v = np.asarray(ms_list) * 1e3
    return {"p10": round(float(np.percentile(v, 10)), 2), "median": round(float(np.median(v)), 2),
            "p90": round(float(np.percentile(v, 90)), 2), "n": int(v.size)}


COLD_BYTES = 512 << 20  # written between cold forwards: twice the 256 MB Infinity Cache, 16 x the L2s


def measure(svdq, torch, wl_name, ydt, steps, warmup, warm_s, compare, log_prefix="", dist=False):
    """Time one workload: the forward (kernel 1 + kernel 2) over `steps` steps after at
    least `warmup` steps and `warm_s` seconds of warm-up, per-kernel HIP-event durations,
    (compare) the rank-0 and unfused forwards in alternating blocks, and (dist) single
    forwards one by one, warm (back to back) and cold (after a 512 MiB write that evicts
    the packed weights and the activations from the L2 and Infinity caches), as
    p10 / median / p90."""
    from bit_diffusion_model_amd.workloads import make

    dev = "cuda:0"
    wl = make(wl_name)
    M, K, N = wl.M, wl.K, wl.N
    fmt = svdq.FMT[wl.fmt]
    log(f"[bench]{log_prefix} workload {wl_name} M={M} K={K} N={N} r={wl.total_rank} fmt={wl.fmt}; packing on host")
    t0 = time.perf_counter()
    hp = svdq.pack_weights(wl.W, svdq.act_absmax(wl.calib), wl.alpha, wl.rank, fmt)
    if wl.lora_A is not None:
        hp = svdq.concat_lora(hp, wl.lora_A, wl.lora_B)
    pack_s = time.perf_counter() - t0
    log(f"[bench]{log_prefix} pack {pack_s:.1f} s (offline, untimed)")
    lay = svdq.PackedLinear.from_host_pack(hp, dev)
    lay0 = svdq.PackedLinear(K, N, 0, fmt, hp.inv_s, hp.L1t[:0], hp.L2[:0], hp.qW, hp.sW, dev)
    r = hp.rank
    X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.float32 if ydt == svdq.F32 else torch.bfloat16, device=dev)
    ws = lay.workspace(M)
    ws0 = lay0.workspace(M)

    def step():
        lay.forward(X, ydt, Y, ws)

    # warm-up: at least `warmup` steps and at least `warm_s` seconds (the clocks take a few
    # tens of ms to settle)
    n, t0 = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < warm_s:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    log(f"[bench]{log_prefix} warmup {n} steps ({time.perf_counter() - t0:.2f} s); timing {steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    ops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
    tops = ops / (ms * 1e-3) / 1e12
    log(f"[bench]{log_prefix} {ms:.4f} ms/step (wall {wall / steps * 1e3:.4f}), {tops:.1f} TOPS")

    # per-kernel durations, launched exactly as inside svdq_linear_forward (activation
    # side in MMA form), with HIP events on the stream the kernels are launched on (torch's
    # current stream, which the binding passes to the library)
    qX, sX, la = lay.alloc_act(M, svdq.ACT_MMA)
    gws = lay.gemm_workspace(M, svdq.ACT_MMA)
    nrep = max(steps, 10)
    k1_parts = lay.forward_k1_parts(M)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4 * nrep)]
    for i in range(nrep):
        e[4 * i].record()
        lay.quantize_act(X, (qX, sX, la), form=svdq.ACT_MMA)
        e[4 * i + 1].record()
        lay.gemm(qX, sX, la, ydt, Y, form=svdq.ACT_MMA, workspace=gws)
        e[4 * i + 2].record()
        if k1_parts > 1:
            step()
        e[4 * i + 3].record()
    torch.cuda.synchronize()
    t_k1 = float(np.mean([e[4 * i].elapsed_time(e[4 * i + 1]) for i in range(nrep)])) * 1e-3
    t_k2 = float(np.mean([e[4 * i + 1].elapsed_time(e[4 * i + 2]) for i in range(nrep)])) * 1e-3
    t_k1_one_pass = t_k1
    if k1_parts > 1:
        # the forward cuts kernel 1 along K (no entry point launches that form alone): its
        # share of the forward is the forward's time less kernel 2's
        t_fwd = float(np.mean([e[4 * i + 2].elapsed_time(e[4 * i + 3]) for i in range(nrep)])) * 1e-3
        t_k1 = t_fwd - t_k2
    # low-rank overhead: the layer against a rank-0 layer with the same codes, and against
    # the unfused baseline (the low-rank branch as kernels of its own), timed in alternating
    # blocks of 20 forwards (medians of 5), so all three see the same clocks
    fr, f0, fu = [], [], []
    for _ in range(5 if compare else 0):
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

    fwd_dist = None
    if dist:
        nw, nc = 100, 20
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nw)]
        for i in range(nw):
            ev[2 * i].record()
            step()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        warm_ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(nw)]
        scratch = torch.empty(COLD_BYTES, dtype=torch.uint8, device=dev)
        cold_ms = []
        for i in range(nc):
            scratch.fill_(i & 255)
            ev[0].record()
            step()
            ev[1].record()
            torch.cuda.synchronize()
            cold_ms.append(ev[0].elapsed_time(ev[1]))
        del scratch
        fwd_dist = {"warm_fwd_us": percentiles_us(warm_ms), "cold_fwd_us": percentiles_us(cold_ms),
                    "cold_eviction": f"{COLD_BYTES >> 20} MiB written before each cold forward"}
        log(f"[bench]{log_prefix} single forwards: warm {fwd_dist['warm_fwd_us']}, cold {fwd_dist['cold_fwd_us']}")

    G = lay.group
    k2_ops = float(M) * N * (2.0 * K + 2.0 * r)
    k1_bytes = k1_algorithmic_bytes(M, K, G, r, fmt == svdq.INT4_G64)
    k2_tops = k2_ops / t_k2 / 1e12
    res = dict(wl=wl, M=M, K=K, N=N, r=r, fmt=fmt, ms=ms, tops=tops, t_k1=t_k1, t_k2=t_k2, k2_tops=k2_tops,
               k1_bytes=k1_bytes, warm_steps=n)
    res["kernels"] = {
        "k1_us": round(t_k1 * 1e6, 2), "k2_us": round(t_k2 * 1e6, 2), "k1_forward_parts": k1_parts,
        "k1_one_pass_us": round(t_k1_one_pass * 1e6, 2),
        "k1_GBps": round(k1_bytes / t_k1 / 1e9, 1), "k1_hbm_frac": round(k1_bytes / t_k1 / 1e9 / PEAK_HBM_GBS, 4),
        "k2_TOPS": round(k2_tops, 2),
        # the INT4 contraction runs on the FP6 scaled MFMA (10.1 PF dense); against the
        # INT8 peak (5.0 POP/s) that the INT4 format would use on an int8 matrix core
        "k2_frac_fp6_fp4_peak": round(k2_tops / PEAK_MFMA_FP4_TOPS, 4),
        # against the peak of the matrix-core instruction kernel 2 runs (FP6/FP4 for INT4 and
        # MXFP4, fp16 for NVFP4)
        "k2_mfma_peak": PEAK_BF16_TOPS if fmt == svdq.NVFP4_G16 else PEAK_MFMA_FP4_TOPS,
        "k2_frac_of_mfma_peak": round(k2_tops / (PEAK_BF16_TOPS if fmt == svdq.NVFP4_G16 else PEAK_MFMA_FP4_TOPS), 4),
        "k2_frac_int8_peak": round(k2_tops / PEAK_INT8_TOPS, 4) if fmt == svdq.INT4_G64 else None,
        "rank0_ms": rnd(ms0, 5), "fwd_ms_paired": rnd(ms_r, 5), "lowrank_overhead": rnd(ms_r / ms0 - 1.0, 4),
        "unfused_ms": rnd(ms_u, 5), "unfused_lowrank_overhead": rnd(ms_u / ms0 - 1.0, 4),
        "host_pack_s": round(pack_s, 2)}
    if fwd_dist:
        res["kernels"].update(fwd_dist)
    return res


def measure_mlp(svdq, torch, steps, warm_s):
    """The chained FLUX.1 MLP pair (C2chain: 4608 tokens, 3072 -> 12288 -> 3072, rank 32,
    INT4): svdq_mlp_forward chained against separate (two forwards, fc1 with the GELU
    output), timed in alternating blocks of 20, and the chained step's kernels one by one
    with HIP events on the launch stream."""
    from bit_diffusion_model_amd.workloads import make_mlp

    dev = "cuda:0"
    d = make_mlp("C2chain")
    M = d.M
    log(f"[bench] [mlp] pair M={M} {d.fc1.K} -> {d.fc1.N} -> {d.fc2.N}; packing on host")
    lays = []
    for wl in (d.fc1, d.fc2):
        hp = svdq.pack_weights(wl.W, svdq.act_absmax(wl.calib), wl.alpha, wl.rank, svdq.INT4_G64)
        lays.append(svdq.PackedLinear.from_host_pack(hp, dev))
    pair = svdq.MlpPair(*lays)
    X = torch.from_numpy(d.fc1.X.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((M, d.fc2.N), dtype=torch.float32, device=dev)
    wsc, wss = pair.workspace(M, svdq.MLP_CHAINED), pair.workspace(M, svdq.MLP_SEPARATE)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(5):
            pair.forward(X, svdq.F32, Y, wsc, svdq.MLP_CHAINED)
            pair.forward(X, svdq.F32, Y, wss, svdq.MLP_SEPARATE)
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tc, ts = [], []
    for _ in range(max(steps // 20, 3)):
        for mode, ws, out in ((svdq.MLP_CHAINED, wsc, tc), (svdq.MLP_SEPARATE, wss, ts)):
            ev0.record()
            for _ in range(20):
                pair.forward(X, svdq.F32, Y, ws, mode)
            ev1.record()
            torch.cuda.synchronize()
            out.append(ev0.elapsed_time(ev1) / 20)
    # the chained path's kernels one by one
    fc1, fc2 = pair.fc1, pair.fc2
    a1 = fc1.alloc_act(M, svdq.ACT_MMA)
    qX2, sX2, la2 = fc2.alloc_act(M, svdq.ACT_MMA)
    part = torch.empty(((fc2.K // 128) * M * svdq.r16(fc2.rank),), dtype=torch.float32, device=dev)
    gws = fc2.gemm_workspace(M, svdq.ACT_MMA)
    nrep = 20
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5 * nrep)]
    for i in range(nrep):
        e[5 * i].record()
        fc1.quantize_act(X, a1, form=svdq.ACT_MMA)
        e[5 * i + 1].record()
        pair.chain_gemm(*a1, M, out=(qX2, sX2, part, None))
        e[5 * i + 2].record()
        pair.chain_reduce(part, M, out=la2)
        e[5 * i + 3].record()
        fc2.gemm(qX2, sX2, la2, svdq.F32, out=Y, form=svdq.ACT_MMA, workspace=gws)
        e[5 * i + 4].record()
    torch.cuda.synchronize()
    us = [float(np.median([e[5 * i + k].elapsed_time(e[5 * i + k + 1]) for i in range(nrep)])) * 1e3 for k in range(4)]
    ms_c, ms_s = float(np.median(tc)), float(np.median(ts))
    ops = sum(2.0 * M * l.N * l.K + 2.0 * M * l.rank * (l.K + l.N) for l in (fc1, fc2))
    log(f"[bench] [mlp] chained {ms_c:.4f} ms, separate {ms_s:.4f} ms")
    return {"workload": "FLUX.1 MLP pair, chained (fc1 -> GELU -> fc2)", "M": M, "K1": fc1.K, "N1": fc1.N,
            "N2": fc2.N, "rank": [fc1.rank, fc2.rank], "chained_ms": round(ms_c, 5), "separate_ms": round(ms_s, 5),
            "chained_TOPS": round(ops / (ms_c * 1e-3) / 1e12, 2), "separate_TOPS": round(ops / (ms_s * 1e-3) / 1e12, 2),
            "chained_speedup": round(ms_s / ms_c, 4),
            "chained_kernels_us": {"fc1_k1": round(us[0], 2), "fc1_k2_chained": round(us[1], 2),
                                   "lora_partials_sum": round(us[2], 2), "fc2_k2": round(us[3], 2)}}


def measure_w4a16(svdq, torch, steps, warm_s, w4a4_ms, mxfp4_ms):
    """The 4-bit weight-only baseline (svdq_w4a16_gemm) on the QKV shape: W's own INT4 g64
    codes upcast to bf16 inside the kernel, bf16 MFMA, fp32 Y; the W4A4 layer's step time
    over it is the layer-level analogue of the pages' speed-up over a weight-only baseline.
    For context, a library bf16 GEMM (torch.matmul, hipBLASLt) on weights upcast beforehand,
    which reads 16-bit weights and does no upcast: the floor of any weight-only layer."""
    from bit_diffusion_model_amd.workloads import make

    dev = "cuda:0"
    wl = make("C1")
    M, K, N = wl.M, wl.K, wl.N
    lay = svdq.WeightOnlyLinear.from_weights(wl.W, dev)
    X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    # bf16(s q) [K][N] from the layer's own codes and scales, for the library GEMM only
    q = lay.qW.to(torch.int32)
    nib = torch.stack([q & 15, q >> 4], -1).reshape(N, K)
    qv = torch.where(nib >= 8, 8 - nib, nib).float()
    Wd = (qv.T * lay.sW.view(torch.float16).float().repeat_interleave(64, 0)).to(torch.bfloat16).contiguous()
    Yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fk = lambda: lay.forward(X, svdq.F32, Y)
    fl = lambda: torch.matmul(X, Wd, out=Yb)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(5):
            fk()
            fl()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tk, tl = [], []
    for _ in range(max(steps // 20, 3)):
        for f, out in ((fk, tk), (fl, tl)):
            ev0.record()
            for _ in range(20):
                f()
            ev1.record()
            torch.cuda.synchronize()
            out.append(ev0.elapsed_time(ev1) / 20)
    ms, ms_l = float(np.median(tk)), float(np.median(tl))
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    log(f"[bench] [w4a16] {ms:.4f} ms ({tf:.1f} TFLOP/s); library bf16 GEMM {ms_l:.4f} ms")
    return {"workload": "FLUX.1 QKV projection, 4-bit weight-only (W4A16) baseline: INT4 g64 fp16 scales "
                        "upcast to bf16 in the kernel, bf16 MFMA, fp32 output",
            "M": M, "K": K, "N": N, "ms": round(ms, 5), "TFLOPs": round(tf, 2),
            "frac_bf16_peak": round(tf / PEAK_BF16_TOPS, 4),
            "w4a4_int4_speedup": round(ms / w4a4_ms, 4) if w4a4_ms else None,
            "w4a4_mxfp4_speedup": round(ms / mxfp4_ms, 4) if mxfp4_ms else None,
            "library_bf16_gemm_ms": round(ms_l, 5),
            "library_bf16_gemm_TFLOPs": round(flops / (ms_l * 1e-3) / 1e12, 2)}


def k1_sweep(svdq, torch):
    """Kernel 1 alone (svdq_quantize_act_lora_down, MMA form) against the token count, per
    format, at K = 3072: random N(0,1) bf16 tokens, unit smoothing factors and random bf16
    down-projection factors (kernel 1's work does not depend on the values).  Best of 5
    blocks of 50 back-to-back launches, HIP events on the launch stream, in us."""
    rng = np.random.default_rng(7)
    K, N = 3072, 256

    def bf(a):
        return ((a.astype(np.float32).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)

    def layer(rank, fmt):
        L1t = bf(rng.standard_normal((rank, K)) * 0.02) if rank else None
        L2 = bf(rng.standard_normal((rank, N)) * 0.02) if rank else None
        qW = np.zeros((K, N // 2), np.uint8)
        sW = {svdq.INT4_G64: np.ones((K // 64, N), np.float16).view(np.uint16),
              svdq.MXFP4_G32: np.full((K // 32, N), 127, np.uint8),
              svdq.NVFP4_G16: np.full((K // 16, N), 0x38, np.uint8)}[fmt]
        return svdq.PackedLinear(K, N, rank, fmt, np.ones(K, np.float32), L1t, L2, qW, sW)

    stream = torch.cuda.current_stream()
    res = {}
    for name, rank, fmt in (("int4_r32", 32, svdq.INT4_G64), ("int4_r0", 0, svdq.INT4_G64),
                            ("mxfp4_r32", 32, svdq.MXFP4_G32), ("nvfp4_r32", 32, svdq.NVFP4_G16)):
        lay = layer(rank, fmt)
        row = {}
        for M in (256, 2048, 4096, 4608, 8192, 9216):
            X = torch.randn(M, K, device="cuda:0").to(torch.bfloat16).view(torch.int16)
            bufs = lay.alloc_act(M, svdq.ACT_MMA)
            for _ in range(20):
                lay.quantize_act(X, bufs, form=svdq.ACT_MMA)
            best = float("inf")
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(50):
                    lay.quantize_act(X, bufs, form=svdq.ACT_MMA)
                e1.record(stream)
                e1.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1000 / 50)
            row[str(M)] = round(best, 2)
            log(f"[k1 sweep] {name} M={M} ({(M + 15) // 16} blocks of 16 tokens): {best:.2f} us")
            del X, bufs
        res[name] = row
    return {"k1_sweep_us": res, "K": K, "blocks": "ceil(M / 16), 8 waves each",
            "note": "kernel 1 alone, MMA form, best of 5 x 50 back-to-back launches"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="minimum warm-up wall time, whatever --warmup says (clocks settle in tens of ms)")
    ap.add_argument("--workload", default="C1", choices=list(WORKLOADS))
    ap.add_argument("--ydtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--cpu-rows", type=int, default=4608)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the rank-0 and unfused comparison forwards (counter runs: only the "
                         "timed layer's kernels are dispatched)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other FLUX workloads (MLP fc1, fc2, MXFP4, batch 2 + LoRA, the chained "
                         "MLP pair)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain device copy of 512 MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="compute kernel 1's and kernel 2's HBM bytes per launch from two rocprofv3 "
                         "--pmc CSVs (FETCH_SIZE, WRITE_SIZE) of runs made with --calib-copy, write the "
                         "summary JSON, and exit")
    ap.add_argument("--k1-sweep", action="store_true",
                    help="time kernel 1 alone per format against the token count (K = 3072), print one "
                         "JSON line and exit")
    ap.add_argument("--write-counters", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"),
                    help="summarise two rocprofv3 --pmc utilisation passes of kernels 1 and 2 (MFMA and "
                         "VALU busy, co-issue, LDS, L2), write the summary JSON, and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_counters:
        write_counters(*args.write_counters, workload=args.workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU: the layer shards along tokens with no "
                                   "exchange step, and only the one-GPU share is implemented and timed; "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import torch
    from bit_diffusion_model_amd import svdq

    svdq.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.k1_sweep:
        print(json.dumps(k1_sweep(svdq, torch)), flush=True)
        return
    ydt = svdq.F32 if args.ydtype == "f32" else svdq.BF16
    m = measure(svdq, torch, args.workload, ydt, args.steps, args.warmup, args.warm_seconds, not args.no_compare,
                dist=not args.no_compare)
    fmt, M, K, N, r = m["fmt"], m["M"], m["K"], m["N"], m["r"]
    k2_tops = m["k2_tops"]
    peak = PEAK_MFMA_FP4_TOPS  # both formats run the FP6 / FP4 scaled MFMA (10.1 PF dense)
    traffic = traffic_entry() if args.workload == "C1" and ydt == svdq.F32 else None
    out = {
        "metric": METRIC, "value": round(m["tops"], 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(m["ms"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4" if fmt == svdq.INT4_G64 else "fp4-e2m1", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "M": M, "K": K, "N": N, "rank": r,
                   "format": {svdq.INT4_G64: "INT4 g64 fp16 scales", svdq.MXFP4_G32: "MXFP4 g32 E8M0 scales",
                              svdq.NVFP4_G16: "NVFP4-style g16 E4M3 + fp32 tensor scales"}[fmt],
                   "output": args.ydtype, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(k2_tops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(k2_tops / peak, 4), "traffic": traffic,
                     "kernel": "kernel 2 (W4A4 GEMM + rescale + low-rank up projection), "
                               + ("INT4 on the FP6 scaled MFMA" if fmt == svdq.INT4_G64 else "MXFP4 scaled MFMA"),
                     "frac_vs_int8_peak": (round(k2_tops / PEAK_INT8_TOPS, 4) if fmt == svdq.INT4_G64 else None)},
        "kernels": m["kernels"],
    }
    if not args.no_others:
        others = {}
        for name in ("C2a", "C2b", "C3", "C4", "C1nv"):
            if name == args.workload:
                continue
            o = measure(svdq, torch, name, ydt, 50, 20, 0.1, not args.no_compare, log_prefix=f" [{name}]")
            others[name] = {"workload": WORKLOADS[name], "M": o["M"], "K": o["K"], "N": o["N"], "rank": o["r"],
                            "ms_per_step": round(o["ms"], 5), "TOPS": round(o["tops"], 2),
                            "k2_frac_fp6_fp4_peak": o["kernels"]["k2_frac_fp6_fp4_peak"], **o["kernels"]}
            del o
            torch.cuda.empty_cache()
        out["workloads"] = others
        out["mlp_pair"] = measure_mlp(svdq, torch, 100, 0.2)
        out["w4a16"] = measure_w4a16(svdq, torch, 100, 0.2, m["ms"] if args.workload == "C1" else None,
                                     others["C3"]["ms_per_step"] if "C3" in others else None)
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} tokens")
        out["cpu_baseline"] = cpu_baseline(args.workload, min(args.cpu_rows, M))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
