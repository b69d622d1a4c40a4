"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and casts them to storage dtypes.  It
holds none of the layer's arithmetic (no routing, no GEMM, no activation), so
both the HIP path and the CPU oracle can take their inputs from it.

Workloads follow the shapes the pages quote for the Mega MoE layer
(Qwen3-30B-A3B: 128 experts, top-8 routing, 16,384 tokens per GPU; Qwen3-235B-
A22B at sequence length 16384), with everything else synthetic:

* x, dout ~ N(0, 1)
* W_gate_up [E, 2I, d] ~ N(0, 1/sqrt(d)),  W_down [E, d, I] ~ N(0, 1/sqrt(I))
* router logits ~ N(0, 1) (+ a per-expert bias for the skewed workloads)

Random streams: ``SeedSequence(seed).spawn(6)`` gives one stream each for
x, logits, bias, W_gate_up, W_down and dout.  The two weight streams are split
again into one child per expert so experts can be drawn in parallel threads;
the values do not depend on the number of threads.  Every tensor is drawn in
float32 and rounded once (round-to-nearest-even) to its storage dtype by
torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# Zipf exponent and temperature of the skewed router bias (fp8 stress
# workload).  The temperature was calibrated once against the oracle's routing
# so that the hottest expert receives about 10x the mean load (see
# tests/golden/calibrate_skew.py, which reproduces it); the four lowest-ranked
# experts get a bias that rules them out, so they receive no token.
ZIPF_S = 1.2
SKEW_TAU = 0.44
SKEW_EMPTY = 4
SKEW_EMPTY_BIAS = -1.0e4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    dtype: str            # storage dtype of x, weights, outputs, grads: "f32" | "bf16"
    logits_dtype: str     # "f32" | "bf16"
    precision: str        # "native" | "fp8_block" | "mxfp8" | "fp8_bwd"
    bias: str             # "none" | "normal" | "zipf"
    bias_std: float = 0.0

    @property
    def R(self) -> int:
        return self.T * self.k

    def flops_fwd(self) -> float:
        return 6.0 * self.R * self.d * self.I

    def flops_bwd(self) -> float:
        return 12.0 * self.R * self.d * self.I

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 128, 64, 8, 2, 128, "f32", "f32", "native", "none"),
    "q30b_t4096": Workload("q30b_t4096", 4096, 2048, 128, 8, 768, "bf16", "bf16", "native", "none"),
    "q30b": Workload("q30b", 16384, 2048, 128, 8, 768, "bf16", "bf16", "native", "none"),
    # one GPU's share of the q30b layer under 8-way expert parallelism: the
    # 16 experts it holds and the 131,072 rows the dispatch exchange brings
    # it, each row its own token (k = 1), about 8192 rows per expert
    "q30b_ep8": Workload("q30b_ep8", 131072, 2048, 16, 1, 768, "bf16", "bf16", "native", "none"),
    "q235b": Workload("q235b", 16384, 4096, 128, 8, 1536, "bf16", "bf16", "native", "normal", 0.5),
    "fp8_skew": Workload("fp8_skew", 16384, 4096, 128, 8, 1536, "bf16", "bf16", "fp8_block", "zipf"),
    # the same skewed layer in MXFP8 (32-value blocks, power-of-two scales)
    "mxfp8_skew": Workload("mxfp8_skew", 16384, 4096, 128, 8, 1536, "bf16", "bf16", "mxfp8", "zipf"),
    # bf16 forward, blockwise fp8 backward
    "fp8_bwd_skew": Workload("fp8_bwd_skew", 16384, 4096, 128, 8, 1536, "bf16", "bf16", "fp8_bwd", "zipf"),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    names = ["x", "logits", "bias", "w_gate_up", "w_down", "dout"]
    return dict(zip(names, ss.spawn(len(names))))


def _normal(seq: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(_TORCH_DTYPE[dtype])


def _expert_weights(seq, E, rows, cols, std, dtype, threads) -> torch.Tensor:
    out = torch.empty((E, rows, cols), dtype=_TORCH_DTYPE[dtype])
    children = seq.spawn(E)

    def one(e):
        out[e].copy_(_cast(_normal(children[e], (rows, cols), std), dtype))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(E)))
    return out


def router_bias(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per-expert router bias [E] (float32) for the workload's bias recipe."""
    seq = _streams(seed)["bias"]
    if wl.bias == "none":
        return np.zeros(wl.E, np.float32)
    if wl.bias == "normal":
        return _normal(seq, (wl.E,), wl.bias_std)
    if wl.bias == "zipf":
        return zipf_bias(wl.E, seq, SKEW_TAU)
    raise ValueError(wl.bias)


def zipf_bias(E: int, seq, tau: float) -> np.ndarray:
    """b_e = tau * log p_rank(e), p_r proportional to r^-ZIPF_S, rank a seeded
    permutation of 1..E; the SKEW_EMPTY lowest-ranked experts get a bias that
    keeps them out of every top-k."""
    g = np.random.Generator(np.random.PCG64(seq))
    rank = g.permutation(E) + 1                       # rank of expert e, 1..E
    logp = -ZIPF_S * np.log(rank.astype(np.float64))
    logp -= np.log(np.sum(np.arange(1, E + 1, dtype=np.float64) ** -ZIPF_S))
    b = (tau * logp).astype(np.float32)
    b[rank > E - SKEW_EMPTY] = np.float32(SKEW_EMPTY_BIAS)
    return b


def make_logits(wl: Workload, seed: int = 0, T: int | None = None,
                bias: np.ndarray | None = None) -> torch.Tensor:
    T = wl.T if T is None else T
    raw = _normal(_streams(seed)["logits"], (wl.T, wl.E))[:T]
    b = router_bias(wl, seed) if bias is None else bias
    return _cast(np.ascontiguousarray(raw + b[None, :]), wl.logits_dtype)


def make_inputs(wl: Workload, seed: int = 0, threads: int = 8,
                with_dout: bool = True) -> dict:
    """All inputs of one layer call as CPU torch tensors in storage dtypes.

    Keys: x [T,d], logits [T,E], w_gate_up [E,2I,d], w_down [E,d,I],
    dout [T,d] (if with_dout).
    """
    s = _streams(seed)
    out = {
        "x": _cast(_normal(s["x"], (wl.T, wl.d)), wl.dtype),
        "logits": make_logits(wl, seed),
        "w_gate_up": _expert_weights(s["w_gate_up"], wl.E, 2 * wl.I, wl.d,
                                     1.0 / math.sqrt(wl.d), wl.dtype, threads),
        "w_down": _expert_weights(s["w_down"], wl.E, wl.d, wl.I,
                                  1.0 / math.sqrt(wl.I), wl.dtype, threads),
    }
    if with_dout:
        out["dout"] = _cast(_normal(s["dout"], (wl.T, wl.d)), wl.dtype)
    return out


def random_topk(T: int, E: int, k: int, seed: int = 0):
    """Ids-in mode inputs drawn independently of any router: k distinct expert
    ids per token (int32 [T,k], a random k-subset in random order) and
    positive weights (float32 [T,k])."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    ids = g.permuted(np.tile(np.arange(E, dtype=np.int32), (T, 1)), axis=1)[:, :k]
    w = g.random((T, k)).astype(np.float32) + np.float32(0.05)
    return torch.from_numpy(np.ascontiguousarray(ids)), torch.from_numpy(w)
