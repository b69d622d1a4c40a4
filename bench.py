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
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer fwd+bwd ms and TFLOP/s (MFMA util %), Qwen3-30B-A3B shape T=16384"


def kernel_work(wl):
    """Algorithmic work per launch of each kernel: ('flop'|'byte', amount)."""
    R, d, I, T, k, E = wl.R, wl.d, wl.I, wl.T, wl.k, wl.E
    es = 2 if wl.dtype == "bf16" else 4
    return {
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


def cpu_baseline(wl, inp: dict, tokens: int):
    """The oracle (fp64 numpy) on the first `tokens` tokens of the workload,
    all experts, forward + backward; rate in TFLOP/s of algorithmic work."""
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
    t0 = time.perf_counter()
    rt = O.route(lg, wl.k, wl.E)
    fw = O.forward(x, rt, Wgu, Wd)
    O.backward(dout, rt, Wgu, Wd, fw, logits=lg)
    dt = time.perf_counter() - t0
    flops = sub.flops_fwd() + sub.flops_bwd()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {tokens} of {wl.T} tokens of the {wl.name} workload, all {wl.E} experts, "
                      f"fwd+bwd in float64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q30b", choices=sorted(S.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer: this build runs on exactly one GPU "
              "(expert-parallel exchange across GPUs is not built); use --gpus 1", file=sys.stderr)
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
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=dt,
                       logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=dev)

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

    flops = wl.flops_fwd() + wl.flops_bwd()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    work = kernel_work(wl)
    kernels = {}
    for name, (n, tot) in kstats.items():
        avg = tot / max(n, 1)
        entry = {"launches_per_step": n / args.steps, "avg_ms": avg}
        if name in work:
            kind, amt = work[name]
            if kind == "flop":
                entry["tflops"] = amt / (avg * 1e-3) / 1e12
                entry["mfma_frac"] = entry["tflops"] / PEAK_BF16_TFLOPS
            else:
                entry["gbs"] = amt / (avg * 1e-3) / 1e9
                entry["hbm_frac"] = entry["gbs"] / PEAK_HBM_GBS
        kernels[name] = entry
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
    kind, amt = work[dom]
    avg = kernels[dom]["avg_ms"]
    if kind == "flop":
        roof = {"kernel": dom, "bound": "mfma", "achieved": amt / (avg * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": amt / (avg * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
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
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: MoE layer fwd+bwd, T={wl.T} tokens, d={wl.d}, E={wl.E}, "
                               f"top-{wl.k}, I={wl.I}, {wl.dtype}, {wl.precision}",
                   "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "I": wl.I, "precision": wl.precision},
        "mfma_util": tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": float(np.median(fwd_ms)),
        "bwd_ms": float(np.median(bwd_ms)),
        "fwd_ms_mean": float(np.mean(fwd_ms)),
        "bwd_ms_mean": float(np.mean(bwd_ms)),
        "two_fwd_plus_bwd_ms": float(2 * np.median(fwd_ms) + np.median(bwd_ms)),
        "gemm_ms_per_step": gemm_ms,
        "gemm_mfma_util": (wl.flops_fwd() + wl.flops_bwd()) / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, inp, min(args.cpu_tokens, wl.T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
