"""Benchmark of the fused MoE layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q30b]

A step is one full pass of the layer on one batch: routing (top-k, counts,
offsets, token sort), gathered gate/up GEMM + SwiGLU, down GEMM, combine, and
the whole backward (top-k-weight and logit gradients, down dgrad/wgrad,
SwiGLU backward, gate/up dgrad/wgrad, dx reduction).  The default workload is
the Qwen3-30B-A3B layer shape at 16,384 tokens (T=16384, d=2048, E=128, k=8,
I=768, bf16), with synthetic inputs already resident in HBM.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the step
(18*T*k*d*I flop per fwd+bwd); `roofline` rates the dominant kernel against
the MI355X dense-bf16 MFMA peak from per-kernel HIP events recorded on the
launch stream during the timed steps; `cpu_baseline` is the CPU oracle timed
on a bounded token sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector (the float32 path runs on FMA units)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer fwd+bwd ms and TFLOP/s (MFMA util %), Qwen3-30B-A3B shape T=16384"
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "combine_top_route_amd", "csrc")

# rocprofv3 kernel name (template instance) -> the library's launch name
KERNEL_SITES = [
    ("rows_gemm_kernel<1, 1, 0>(", "gemm_gateup_fwd"), ("rows_gemm_kernel<0, 0, 0>(", "gemm_down_fwd"),
    ("rows_gemm_kernel<0, 2, 1>(", "gemm_down_dgrad"), ("rows_gemm_kernel<0, 2, 0>(", "gemm_gateup_dgrad"),
    ("rows_persist_kernel<1, 1, 0>(", "gemm_gateup_fwd"), ("rows_persist_kernel<0, 0, 0>(", "gemm_down_fwd"),
    ("rows_persist_kernel<0, 2, 1>(", "gemm_down_dgrad"), ("rows_persist_kernel<0, 2, 0>(", "gemm_gateup_dgrad"),
    ("wgrad_kernel<0>(", "gemm_down_wgrad"), ("wgrad_kernel<1>(", "gemm_gateup_wgrad"),
    ("wgrad_persist_kernel<0>(", "gemm_down_wgrad"), ("wgrad_persist_kernel<1>(", "gemm_gateup_wgrad"),
    ("rows8_kernel<1, 0, ", "gemm_gateup_fwd"), ("rows8_kernel<0, 0, ", "gemm_down_fwd"),
    ("rows8_kernel<2, 2, ", "gemm_down_dgrad"), ("rows8_kernel<0, 1, ", "gemm_gateup_dgrad"),
    ("wgrad8_kernel<0, ", "gemm_down_wgrad"), ("wgrad8_kernel<1, ", "gemm_gateup_wgrad"),
    ("combine_wide_kernel<", "combine + reduce_dx"), ("combine_kernel<", "combine + reduce_dx"),
    ("topk_lane_kernel<", "route_topk"), ("topk_kernel<", "route_topk"), ("count_kernel", "route_count"),
    ("permute_kernel", "permute"), ("permute_scatter_kernel", "permute"),  # before route's scatter_kernel
    ("scan_kernel", "route_scan"), ("scatter_kernel", "route_scatter"), ("schedule_kernel", "route_schedule"),
    ("tok_of_kernel", "route_tok"),
    ("topk_grad_kernel", "topk_grad"), ("swiglu_bwd", "swiglu_bwd"), ("quant_rows_kernel", "quant_x/dout/aw"),
    ("quant_weight_kernel", "quant_w_*"), ("quant_weight_mx_kernel", "quant_w_*"),
    ("quant_tok_kernel", "quant_*_tok"),
]
# source files whose text defines each GEMM kernel (a change voids measured traffic)
KERNEL_SOURCES = {
    "native": ["gemm_bf16.hip", "tile.h", "common.h"],
    "fp8_block": ["gemm_fp8.hip", "tile.h", "common.h"],
    "mxfp8": ["gemm_fp8.hip", "tile.h", "common.h"],
    "fp8_bwd": ["gemm_bf16.hip", "gemm_fp8.hip", "tile.h", "common.h"],
}
FP8 = ("fp8_block", "mxfp8", "fp8_bwd")
FWD_GEMMS = ("gemm_gateup_fwd", "gemm_down_fwd")


def site_of(kernel_name: str) -> str | None:
    for key, site in KERNEL_SITES:
        if key in kernel_name:
            return site
    return None


def mfma_peak(wl, kernel: str | None = None) -> float:
    """MFMA peak of the workload's GEMMs (of one GEMM when kernel is given:
    fp8_bwd runs its forward GEMMs in bf16)."""
    if wl.precision in FP8 and not (wl.precision == "fp8_bwd" and kernel in FWD_GEMMS):
        return PEAK_FP8_TFLOPS
    return PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS


def kernel_work(wl):
    """Algorithmic work per launch of each kernel: ('flop'|'byte', amount)."""
    R, d, I, T, k, E = wl.R, wl.d, wl.I, wl.T, wl.k, wl.E
    es = 2 if wl.dtype == "bf16" else 4
    work = {
        "gemm_gateup_fwd": ("flop", 4.0 * R * d * I),
        "gemm_down_fwd": ("flop", 2.0 * R * d * I),
        "gemm_down_dgrad": ("flop", 2.0 * R * d * I),
        "gemm_down_wgrad": ("flop", 2.0 * R * d * I),
        "gemm_gateup_dgrad": ("flop", 4.0 * R * d * I),
        "gemm_gateup_wgrad": ("flop", 4.0 * R * d * I),
        # read R rows + write T rows + row_of (the rows already carry their weight)
        "combine": ("byte", float(R * d * es + T * d * es + 4 * R)),
        "reduce_dx": ("byte", float(R * d * es + T * d * es + 4 * R)),
        "permute": ("byte", float(T * d * es + R * d * es + 4 * R)),
        "route_topk": ("byte", float(T * E * es + 8 * R)),
    }
    if wl.precision in FP8:
        # bf16 in, one code byte out per element, plus scales: an fp32 scale
        # per 128 values of a row (blockwise) or an E8M0 byte per 32 (MX) --
        # the same 1/32 byte per value; weights: an fp32 scale per 128 x 128
        # block (blockwise) or a byte per 32 values (MX)
        q = lambda n: float(n * 2 + n + n // 32)
        ws = (lambda n: n // 32) if wl.precision == "mxfp8" else (lambda n: 4 * n // 16384)
        # layouts a weight encoder writes: blockwise one (a 128 x 128 block
        # has one scale whichever axis a GEMM contracts, so the data
        # gradients read the forward codes); MX two (its 1 x 32 blocks run
        # along one axis, so the data gradients get a transposed encoding)
        nl = 2 if wl.precision == "mxfp8" else 1
        qw = lambda n: float(n * 2 + nl * (n + ws(n)))
        work.update({
            "quant_x": ("byte", q(T * d)), "quant_dout": ("byte", q(T * d)),
            "quant_aw": ("byte", q(R * I)),
            "quant_w_gate_up": ("byte", qw(E * 2 * I * d)),
            "quant_w_down": ("byte", qw(E * d * I)),
            "quant_dout_tok": ("byte", q(R * d) + 4 * R), "quant_x_tok": ("byte", q(R * d) + 4 * R),
            "quant_aw_tok": ("byte", q(R * I)), "quant_dh_tok": ("byte", q(R * 2 * I)),
        })
    return work


def source_digest(wl) -> str:
    """Digest of the GEMM sources' code, comments removed (a comment edit
    leaves the counters of the committed summaries valid; any code edit
    voids them)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[wl.precision]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(text.encode())
    return h.hexdigest()[:16]


def measured_traffic(wl, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload, or None when there is none or the kernel's
    source changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", f"hbm_traffic_{wl.name}.md")
    if not os.path.exists(path):
        return None
    digest = None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("source digest:"):
                digest = line.split(":", 1)[1].strip()
            if line.startswith("traffic:"):
                parts = dict(p.split("=") for p in line.split()[2:])
                vals[line.split()[1]] = parts
    if digest != source_digest(wl) or kernel not in vals:
        return None
    v = vals[kernel]
    return {"fetch_bytes": float(v["fetch"]), "write_bytes": float(v["write"]),
            "bytes": float(v["fetch"]) + float(v["write"])}


def cpu_baseline(wl, inp: dict, tokens: int):
    """The oracle (fp64 numpy) on the first `tokens` tokens of the workload,
    all experts, forward + backward; rate in TFLOP/s of algorithmic work.

    MXFP8 encodes every expert's two weights in two blockings, a fixed cost
    (minutes in numpy) that no token sample bounds; its sample is instead the
    rows of the two most-loaded experts among the first `tokens` tokens,
    through the oracle's per-expert evaluator (gate/up forward, down dgrad,
    both weight gradients), whose work is 12 rows d I."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    sub = wl.scaled(T=tokens)
    f = lambda t: t[:tokens].double().numpy()
    x, lg, dout = f(inp["x"]), f(inp["logits"]), f(inp["dout"])
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    fp8 = wl.precision in FP8
    recipe = O.MXFP8 if wl.precision == "mxfp8" else O.FP8_BLOCK
    fwd_recipe = O.NO_QUANT if wl.precision == "fp8_bwd" else recipe
    if wl.precision == "mxfp8":
        rt = O.route(lg, wl.k, wl.E)
        top = np.argsort(-rt["counts"], kind="stable")[:2]
        t0 = time.perf_counter()
        for e in top:
            O.expert_weight_grads_fp8(x, dout, rt, Wgu, Wd, int(e), recipe=recipe)
        dt = time.perf_counter() - t0
        rows = int(rt["counts"][top].sum())
        return {"value": 12.0 * rows * wl.d * wl.I / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle",
                "sample": f"rows of experts {[int(e) for e in top]} ({rows} rows) among the first {tokens} "
                          f"tokens of the {wl.name} workload, per-expert fwd gate/up + down dgrad + both "
                          f"weight gradients in float64 numpy emulating MXFP8, {dt:.1f} s"}
    t0 = time.perf_counter()
    rt = O.route(lg, wl.k, wl.E)
    if fp8:
        fw = O.forward_fp8(x, rt, Wgu, Wd, recipe=fwd_recipe)
        O.backward_fp8(dout, rt, Wgu, Wd, fw, logits=lg, recipe=recipe)
    else:
        fw = O.forward(x, rt, Wgu, Wd)
        O.backward(dout, rt, Wgu, Wd, fw, logits=lg)
    dt = time.perf_counter() - t0
    flops = sub.flops_fwd() + sub.flops_bwd()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {tokens} of {wl.T} tokens of the {wl.name} workload, all {wl.E} experts, "
                      f"fwd+bwd in float64 numpy{' emulating the fp8 quantisation' if fp8 else ''}, "
                      f"{dt:.1f} s"}


COPY_BYTES = 1 << 30
# oracle sample per workload: about 10-30 s of float64 numpy on 16 host cores
CPU_SAMPLE_TOKENS = {"q30b": 16384, "q30b_t4096": 4096, "q30b_ep8": 131072, "q235b": 8192, "fp8_skew": 2048,
                     "mxfp8_skew": 2048, "fp8_bwd_skew": 2048}


def gemm_operand_bytes(wl):
    """Bytes each GEMM must move at least once: both operands and the result
    (weights once, activation rows once), in the storage types it reads."""
    R, d, I, T, E = wl.R, wl.d, wl.I, wl.T, wl.E
    a = 1 if wl.precision in FP8 else (2 if wl.dtype == "bf16" else 4)
    o = 2 if wl.dtype == "bf16" else 4
    return {
        "gemm_gateup_fwd": T * d * a + E * 2 * I * d * a + R * 3 * I * o,
        "gemm_down_fwd": R * I * a + E * d * I * a + R * d * o,
        "gemm_down_dgrad": T * d * a + E * d * I * a + 2 * R * 2 * I * o,
        "gemm_down_wgrad": R * d * a + R * I * a + E * d * I * o,
        "gemm_gateup_dgrad": R * 2 * I * a + E * 2 * I * d * a + R * d * o,
        "gemm_gateup_wgrad": R * 2 * I * a + R * d * a + E * 2 * I * d * o,
    }


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


MFMA_COUNTERS = "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT"


def mfma_summary(wl, out: str, pmc_dir: str):
    """Markdown summary of one rocprofv3 --pmc run of MFMA_COUNTERS: per
    launch, the sustained clock, the MFMA units' busy share and LDS activity."""
    import collections
    n = wl.name
    per = collections.defaultdict(dict)
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        site = site_of(r["Kernel_Name"])
        if site is None:
            continue
        key = (site, r.get("Dispatch_Id") or r.get("Correlation_Id"))
        d = per[key]
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = collections.defaultdict(list)
    for (site, _), d in per.items():
        if d.get("GRBM_GUI_ACTIVE", 0) > 0 and d["ns"] > 0:
            cyc = d["GRBM_GUI_ACTIVE"] / 8  # summed over the 8 XCDs
            agg[site].append((d["ns"] / 1e3, cyc / d["ns"], d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * 1024),
                              d.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * 256),
                              d.get("SQ_LDS_BANK_CONFLICT", 0.0) / (cyc * 256)))
    lines = [f"# rocprofv3 summary: MFMA busy cycles, LDS activity and sustained clock, {n} workload "
             f"(T={wl.T}, d={wl.d}, E={wl.E}, k={wl.k}, I={wl.I}, {wl.dtype}, {wl.precision})", "",
             "Commands (repository root, TMPDIR=/tmp):", "",
             f"    rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d {pmc_dir} -o {n} -- python3 bench.py "
             f"--workload {n} --steps 2 --warmup 1 --no-cpu",
             f"    python3 bench.py --workload {n} --mfma-summary {out} {pmc_dir}", "",
             "Per dispatch (one CSV row per dispatch and counter):",
             "- GRBM_GUI_ACTIVE is summed over the 8 XCDs; one XCD's busy cycles are the value / 8.",
             "- clock = (GRBM_GUI_ACTIVE / 8) / (End_Timestamp - Start_Timestamp).",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ((GRBM_GUI_ACTIVE / 8) * 1024 SIMDs).",
             "- LDS active = SQ_LDS_IDX_ACTIVE / ((GRBM_GUI_ACTIVE / 8) * 256 CUs); bank conflicts likewise.",
             "- The clock is meaningful for long dispatches only: GRBM_GUI_ACTIVE also counts launch overhead.", "",
             "| launch | dispatches | avg us | clock GHz | MFMA busy | LDS active | LDS bank conflict |",
             "|---|---|---|---|---|---|---|"]
    for site, v in sorted(agg.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        m = np.mean(np.array(v), axis=0)
        mf = f"{100 * m[2]:.1f}%" if site.startswith("gemm") else "-"
        ghz = f"{m[1]:.2f}" if m[0] >= 50 else "-"  # launch overhead dominates short dispatches
        lines.append(f"| {site} | {len(v)} | {m[0]:.1f} | {ghz} | {mf} | {100 * m[3]:.1f}% | {100 * m[4]:.2f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def rocprof_summary(wl, out: str, stats_dir: str, fetch_dir: str | None = None, write_dir: str | None = None,
                    flags: str = ""):
    """Markdown summary of rocprofv3 output: per-kernel durations from
    --kernel-trace --stats and, given two --pmc runs (FETCH_SIZE, WRITE_SIZE),
    HBM bytes per launch scaled by the same counters on the 1 GiB copy."""
    n = wl.name
    lines = [f"# rocprofv3 summary, {n} workload (T={wl.T}, d={wl.d}, E={wl.E}, k={wl.k}, "
             f"I={wl.I}, {wl.dtype}, {wl.precision})", "",
             "Commands (repository root, TMPDIR=/tmp):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d {stats_dir} -o {n} -- "
             f"python3 bench.py --workload {n} --steps 5 --warmup 2 --no-cpu{flags}"]
    if fetch_dir and write_dir:
        for key, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            lines.append(f"    rocprofv3 --pmc {key} --output-format csv -d {d} -o {n} -- python3 bench.py "
                         f"--workload {n} --steps 2 --warmup 1 --no-cpu --copy-calibration{flags}")
    lines += [f"    python3 bench.py --workload {n}{flags} --rocprof-summary {out} {stats_dir}"
              + (f" {fetch_dir} {write_dir}" if fetch_dir and write_dir else ""), ""]
    stats = _csv_rows(stats_dir, "kernel_stats.csv")
    lines += ["Kernel durations (rocprofv3 --kernel-trace --stats):", "",
              "| launch | kernel | calls | avg us | % GPU time |", "|---|---|---|---|---|"]
    other = 0.0
    for r in sorted(stats, key=lambda r: -float(r["Percentage"])):
        name = r["Name"]
        if site_of(name) is None:  # torch's and the runtime's own kernels
            other += float(r["Percentage"])
            continue
        short = name.replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {site_of(name)} | `{short}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"Left out above: torch's and the runtime's own kernels ({other:.2f}% of GPU time)."]
    if fetch_dir and write_dir:
        per = {}
        for key, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            for r in _csv_rows(d, "counter_collection.csv"):
                if r["Counter_Name"] != key:
                    continue
                site = site_of(r["Kernel_Name"])
                if site is None and "copyBuffer" in r["Kernel_Name"]:  # the runtime's device copy
                    site = "calibration copy"
                if site is None:
                    continue
                per.setdefault(site, {}).setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        cal = per.get("calibration copy")
        if not cal or "FETCH_SIZE" not in cal or "WRITE_SIZE" not in cal:
            raise SystemExit("no calibration copy kernel in the counter runs (bench.py --copy-calibration)")
        # the 1 GiB copies (the calibration copy and the attainable-peak
        # copy, the same size) are the runtime's largest copies; smaller ones
        # move inputs, so the maximum, not the mean
        cal = {key: [max(v)] for key, v in cal.items()}
        f_fetch = COPY_BYTES / float(np.mean(cal["FETCH_SIZE"]))
        f_write = COPY_BYTES / float(np.mean(cal["WRITE_SIZE"]))
        lines += ["", "HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, KiB per "
                      "dispatch), scaled by the counters of a plain 1 GiB copy kernel in the same runs:",
                  f"fetch factor {f_fetch:.4f} (copy read {np.mean(cal['FETCH_SIZE']) / 2**20:.1f} MiB by "
                  f"the counter), write factor {f_write:.4f} (copy wrote "
                  f"{np.mean(cal['WRITE_SIZE']) / 2**20:.1f} MiB).", "",
                  f"source digest: {source_digest(wl)}", "",
                  "| launch | dispatches | fetch MB | write MB | operand MB (minimum) |", "|---|---|---|---|---|"]
        ops = gemm_operand_bytes(wl)
        tr = []
        for site, v in sorted(per.items()):
            if site == "calibration copy" or "FETCH_SIZE" not in v or "WRITE_SIZE" not in v:
                continue
            fb = float(np.mean(v["FETCH_SIZE"])) * f_fetch
            wb = float(np.mean(v["WRITE_SIZE"])) * f_write
            om = ops.get(site)
            lines.append(f"| {site} | {len(v['FETCH_SIZE'])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                         f"{'' if om is None else f'{om / 1e6:.1f}'} |")
            if site.startswith("gemm_"):
                tr.append(f"traffic: {site} fetch={fb:.0f} write={wb:.0f}")
        lines += ["", "Machine-readable (bytes per launch, read by bench.py while the source digest matches):",
                  ""] + tr
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def attainable_peaks(wl, dev, reps: int = 10):
    """Measured attainable peaks on this GPU, for the roofline fractions
    beside the published ones: a large square GEMM through torch (hipBLASLt)
    in bf16, and in fp8 (torch._scaled_mm, unit scales) for the fp8
    workloads, and torch's streaming copy of 1 GiB (bytes read + written;
    the row passes of this library run faster than it, so it is reported,
    not used as a ceiling)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    out = {}
    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    bt = torch.randn((n, n), device=dev).to(torch.bfloat16)
    out["gemm_bf16_tflops"] = 2.0 * n ** 3 / timed(lambda: torch.mm(a, bt.t())) / 1e12
    out["gemm_bf16_shape"] = f"{n}x{n}x{n}, torch.mm (hipBLASLt), B transposed"
    if wl.precision in FP8:
        try:
            a8, b8 = a.to(torch.float8_e4m3fn), bt.to(torch.float8_e4m3fn)
            one = torch.ones((), device=dev)
            out["gemm_fp8_tflops"] = 2.0 * n ** 3 / timed(
                lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)) / 1e12
        except Exception as e:  # an op this torch build does not run on the device
            out["gemm_fp8_error"] = f"{type(e).__name__}: {str(e).splitlines()[0][:200]}"
    del a, bt
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    out["copy_gbs"] = 2.0 * COPY_BYTES / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def library_gemms(wl, layer, x, wgu, wd, steps):
    """The forward GEMM shapes of the layer through torch's own GEMMs, for
    context: torch._grouped_mm over the expert-sorted rows (no gather, no
    SwiGLU, no weighting: plain grouped products at the same offsets), and one
    dense torch.mm with the same FLOPs (all rows against one expert's weight).
    Times are per call from CUDA events over `steps` calls after one warm-up."""
    dt = x.dtype
    R, d, I = wl.R, wl.d, wl.I
    xp = torch.empty((R, d), dtype=dt, device=x.device)
    B.permute(x, layer.routing, wl.k, out=xp)
    offs = layer.routing.offsets[1:].to(torch.int32).contiguous()
    aw = torch.randn((R, I), device=x.device).to(dt)
    cases = {
        "grouped_gateup_fwd": (lambda: torch._grouped_mm(xp, wgu.transpose(1, 2), offs=offs), 4.0 * R * d * I),
        "grouped_down_fwd": (lambda: torch._grouped_mm(aw, wd.transpose(1, 2), offs=offs), 2.0 * R * d * I),
        "dense_gateup_fwd": (lambda: torch.mm(xp, wgu[0].t()), 4.0 * R * d * I),
        "dense_down_fwd": (lambda: torch.mm(aw, wd[0].t()), 2.0 * R * d * I),
    }
    out = {}
    for name, (fn, flop) in cases.items():
        try:
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            b.synchronize()
            ms = a.elapsed_time(b) / steps
            out[name] = {"avg_ms": ms, "tflops": flop / (ms * 1e-3) / 1e12}
        except Exception as e:  # an op this torch build does not run on the device
            out[name] = {"error": f"{type(e).__name__}: {str(e).splitlines()[0][:200]}"}
    del xp, aw
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q30b", choices=sorted(S.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the oracle's CPU sample (default: sized for roughly 10-30 s)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--library-gemms", action="store_true",
                    help="also time the forward GEMM shapes through torch._grouped_mm and torch.mm (context)")
    ap.add_argument("--persistent", action="store_true",
                    help="bf16 GEMMs as persistent kernels (MOE_FLAG_PERSISTENT)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, copy 1 GiB once (a plain copy kernel of known size "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("OUT.md", "PMC_DIR"),
                    help="write the clock / MFMA busy / LDS summary of a rocprofv3 --pmc run of "
                         + MFMA_COUNTERS)
    ap.add_argument("--rocprof-summary", nargs="+", metavar="ARG",
                    help="OUT.md STATS_DIR [FETCH_DIR WRITE_DIR]: write the summary of rocprofv3 "
                         "--kernel-trace --stats output (and of two --pmc runs) for --workload")
    args = ap.parse_args()
    if args.mfma_summary:
        mfma_summary(S.WORKLOADS[args.workload], *args.mfma_summary)
        return
    if args.rocprof_summary:
        rocprof_summary(S.WORKLOADS[args.workload], *args.rocprof_summary,
                        flags=" --persistent" if args.persistent else "")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer on exactly one GPU (the library has no "
              "expert-parallel exchange across GPUs); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    wl = S.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = S.torch_dtype(wl.dtype)
    inp = S.make_inputs(wl, seed=args.seed)
    x = inp["x"].to(dev)
    logits = inp["logits"].to(dev)
    wgu = inp["w_gate_up"].to(dev)
    wd = inp["w_down"].to(dev)
    dout = inp["dout"].to(dev)
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=dt, logits_dtype=S.torch_dtype(wl.logits_dtype),
                       precision=wl.precision, device=dev, persistent=args.persistent)

    def step():
        layer.forward(x, wgu, wd, logits=logits)
        layer.backward(dout, x, wgu, wd)

    B.profile_begin()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    B.profile_end()

    # timed region: K steps, synchronised on both sides; per-kernel HIP events
    # are recorded on the launch stream while it runs
    B.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kstats = B.profile_end()
    ms_per_step = elapsed * 1e3 / args.steps

    # the dispatch alone (moe_permute: each token's row copied to its k
    # expert-sorted rows), outside the layer step, on the step's routing
    xp = torch.empty((wl.R, wl.d), dtype=dt, device=dev)
    B.permute(x, layer.routing, wl.k, out=xp)
    torch.cuda.synchronize()
    B.profile_begin()
    for _ in range(args.steps):
        B.permute(x, layer.routing, wl.k, out=xp)
    torch.cuda.synchronize()
    kstats.update(B.profile_end())
    del xp

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    lib = library_gemms(wl, layer, x, wgu, wd, args.steps) if args.library_gemms and wl.dtype == "bf16" else None
    attain = attainable_peaks(wl, dev)

    # forward alone and backward alone (events around each call)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    fwd_ms, bwd_ms = [], []
    for _ in range(args.steps):
        a, b, c = ev(), ev(), ev()
        a.record()
        layer.forward(x, wgu, wd, logits=logits)
        b.record()
        layer.backward(dout, x, wgu, wd)
        c.record()
        c.synchronize()
        fwd_ms.append(a.elapsed_time(b))
        bwd_ms.append(b.elapsed_time(c))

    # activation checkpointing: forward keeping nothing, then the backward
    # that recomputes the gate/up half from x (moe_backward with saved = NULL)
    del layer
    torch.cuda.empty_cache()
    ac = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=dt, logits_dtype=S.torch_dtype(wl.logits_dtype),
                    precision=wl.precision, device=dev, save=False, persistent=args.persistent)
    ac_ms = []
    for i in range(args.warmup + args.steps):
        a, b = ev(), ev()
        a.record()
        ac.forward(x, wgu, wd, logits=logits)
        ac.backward(dout, x, wgu, wd)
        b.record()
        b.synchronize()
        if i >= args.warmup:
            ac_ms.append(a.elapsed_time(b))
    del ac

    flops = wl.flops_fwd() + wl.flops_bwd()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    work = kernel_work(wl)
    kernels = {}
    for name, (n, tot) in kstats.items():
        avg = tot / max(n, 1)
        # the dispatch is timed on its own, outside the step
        entry = {"launches_per_step": 0.0 if name == "permute" else n / args.steps, "avg_ms": avg}
        if name in work:
            kind, amt = work[name]
            if kind == "flop":
                entry["tflops"] = amt / (avg * 1e-3) / 1e12
                entry["mfma_frac"] = entry["tflops"] / mfma_peak(wl, name)
                att = attain.get("gemm_fp8_tflops" if mfma_peak(wl, name) == PEAK_FP8_TFLOPS
                                 else "gemm_bf16_tflops") if wl.dtype == "bf16" else None
                if att:
                    entry["frac_attainable"] = entry["tflops"] / att
            else:
                entry["gbs"] = amt / (avg * 1e-3) / 1e9
                entry["hbm_frac"] = entry["gbs"] / PEAK_HBM_GBS
                # torch's copy kernel is no ceiling: the row passes here run faster
                entry["frac_of_torch_copy"] = entry["gbs"] / attain["copy_gbs"]
        kernels[name] = entry
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
    kind, amt = work[dom]
    avg = kernels[dom]["avg_ms"]
    if kind == "flop":
        bound = "mfma" if (wl.dtype == "bf16") else "alu"
        roof = {"kernel": dom, "bound": bound, "achieved": amt / (avg * 1e-3) / 1e12,
                "peak": mfma_peak(wl, dom), "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": amt / (avg * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same against the measured attainable peak (a square GEMM of the
    # kernel's dtype through the vendor library)
    att = attain.get("gemm_fp8_tflops" if roof["peak"] == PEAK_FP8_TFLOPS else "gemm_bf16_tflops") \
        if kind == "flop" and wl.dtype == "bf16" else None
    if att:
        roof["attainable"] = att
        roof["frac_attainable"] = roof["achieved"] / att
    tr = measured_traffic(wl, dom)
    roof["traffic"] = None if tr is None else tr["bytes"]
    if tr is not None:
        roof["traffic_detail"] = {**tr, "source": f"profiles/hbm_traffic_{wl.name}.md",
                                  "algorithmic_operand_bytes": gemm_operand_bytes(wl).get(dom)}
    gemm_ms = sum(kernels[k]["avg_ms"] * kernels[k]["launches_per_step"] for k in kernels if k.startswith("gemm"))

    res = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8_block": "fp8_e4m3 (fp32 block scales, fp32 accumulate)",
                  "mxfp8": "fp8_e4m3 (MXFP8: E8M0 scale per 32 values, fp32 accumulate)",
                  "fp8_bwd": "bf16 forward, fp8_e4m3 backward (fp32 block scales)"}.get(
                      wl.precision, "bf16" if wl.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: MoE layer fwd+bwd, T={wl.T} tokens, d={wl.d}, E={wl.E}, "
                               f"top-{wl.k}, I={wl.I}, {wl.dtype}, {wl.precision}",
                   "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "I": wl.I, "precision": wl.precision,
                   "row_gemms": "persistent" if args.persistent else "one tile per work-group"},
        "mfma_util": tflops / mfma_peak(wl),
        "fwd_ms": float(np.median(fwd_ms)),
        "bwd_ms": float(np.median(bwd_ms)),
        "fwd_ms_mean": float(np.mean(fwd_ms)),
        "bwd_ms_mean": float(np.mean(bwd_ms)),
        "two_fwd_plus_bwd_ms": float(2 * np.median(fwd_ms) + np.median(bwd_ms)),
        # measured: forward without saving + backward that recomputes H and Aw
        "recompute_step_ms": float(np.median(ac_ms)),
        "gemm_ms_per_step": gemm_ms,
        "gemm_mfma_util": (wl.flops_fwd() + wl.flops_bwd()) / (gemm_ms * 1e-3) / 1e12 / mfma_peak(wl),
        "roofline": roof,
        "kernels": kernels,
        "attainable": attain,
    }
    if lib is not None:
        res["library_gemms"] = lib
    if not args.no_cpu:
        n = args.cpu_tokens or CPU_SAMPLE_TOKENS.get(wl.name, wl.T)
        print(f"bench: GPU timing done ({ms_per_step:.3f} ms/step); CPU oracle baseline on {min(n, wl.T)} "
              f"tokens", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, inp, min(n, wl.T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
