"""Persistent GEMMs (MOE_FLAG_PERSISTENT: the bf16 row GEMMs and weight
gradients) against the oracle and against the default engine.

With the flag, one work-group per CU walks its XCD's tiles and issues the
next tile's first stage (gathered token rows and weight slice; for a weight
gradient, its first rows of both operands) during the current tile's last K
step ("Prime Intellect's Prime Mega MoE Trains
Giant AI Models 55% Faster", section "One kernel overlaps the pipeline").
Every output row still takes the same MFMAs in the same K order, so all
results must equal the default engine's bit for bit, and the oracle's
within the layer tolerance.  The cases cover K and N tails in every row
GEMM, single-step K loops (d = 64, I = 40), a one-token layer, empty
experts next to a hot one, the bf16 forward of fp8_bwd, the recomputing
backward, and q30b and q235b at full size (bit equality only: the oracle
at those sizes is covered by the full-size parity tests).
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

from gpu_util import TOL, check_floats, check_routing, run_oracle, to_np

pytestmark = pytest.mark.gpu

TINY = S.WORKLOADS["tiny"]
BF = dict(dtype="bf16", logits_dtype="bf16")
CASES = {
    "ragged_tails": TINY.scaled(T=3001, d=2000, E=40, k=6, I=712, **BF),
    "one_k_step": TINY.scaled(T=500, d=64, E=12, k=3, I=40, **BF),
    "one_token": TINY.scaled(T=1, d=128, E=8, k=2, I=128, **BF),
    "fp8_bwd": TINY.scaled(T=600, d=256, E=8, k=2, I=256, precision="fp8_bwd", **BF),
    "min_dims": TINY.scaled(T=333, d=8, E=6, k=2, I=8, **BF),
    "max_d": TINY.scaled(T=40, d=16384, E=4, k=2, I=64, **BF),
    "wide_i": TINY.scaled(T=500, d=136, E=8, k=2, I=648, **BF),
}
NAMES = ("out", "saved", "dx", "dW_gate_up", "dW_down", "d_topk_w", "dlogits")


def _run(wl, inp, persistent, ids=None, w=None, save=True):
    dev = torch.device("cuda", 0)
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=S.torch_dtype(wl.dtype),
                       logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=dev,
                       save=save, persistent=persistent)
    x, wgu, wd = (inp[n].to(dev) for n in ("x", "w_gate_up", "w_down"))
    if ids is None:
        layer.forward(x, wgu, wd, logits=inp["logits"].to(dev))
    else:
        layer.forward(x, wgu, wd, topk_ids=ids.to(dev), topk_w=w.to(dev))
    res = {"out": layer.out.clone()}
    if save:
        res["saved"] = layer.saved.clone()
    for n in ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of"):
        res[n] = getattr(layer.routing, n).clone()
    for n, v in layer.backward(inp["dout"].to(dev), x, wgu, wd).items():
        res[n] = v.clone()
    torch.cuda.synchronize()
    return res


def _bit_equal(a, b, names=NAMES):
    for n in names:
        if n in a and n in b:
            assert torch.equal(a[n], b[n]), f"{n} differs from the default engine"


@pytest.mark.parametrize("case", sorted(CASES))
def test_persistent_matches_oracle_and_default(case):
    wl = CASES[case]
    inp = S.make_inputs(wl, seed=31)
    print(f"persistent case {case}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} I={wl.I} {wl.precision}", flush=True)
    got = _run(wl, inp, True)
    _bit_equal(got, _run(wl, inp, False))
    ref = run_oracle(wl, inp)
    gnp = {n: to_np(v) for n, v in got.items()}
    check_routing(gnp, ref)
    tol = TOL["fp8"] if wl.precision != "native" else TOL[wl.dtype]
    check_floats(gnp, ref, tol)


def test_persistent_empty_and_hot_experts():
    """ids-in routing: 3 of 64 experts take about two thirds of the rows,
    52 are empty, and one expert holds a single row."""
    wl = TINY.scaled(T=2000, d=512, E=64, k=2, I=256, **BF)
    inp = S.make_inputs(wl, seed=32)
    g = torch.Generator().manual_seed(33)
    first = torch.where(torch.rand(wl.T, generator=g) < 0.9, torch.randint(0, 3, (wl.T,), generator=g),
                        torch.randint(3, 12, (wl.T,), generator=g))
    second = (first + 1 + torch.randint(0, 2, (wl.T,), generator=g)) % 12
    ids = torch.stack([first, second], 1).to(torch.int32)
    ids[7, 1] = 40                       # the only row of expert 40
    w = torch.rand(wl.T, wl.k, generator=g)
    print("persistent case empty_and_hot", flush=True)
    got = _run(wl, inp, True, ids, w)
    _bit_equal(got, _run(wl, inp, False, ids, w))
    counts = to_np(got["counts"])
    assert counts[40] == 1 and (counts == 0).sum() >= 50 and counts[:3].sum() > 0.6 * wl.T * wl.k
    ref = run_oracle(wl, inp, ids, w)
    check_floats({n: to_np(v) for n, v in got.items()}, ref, TOL["bf16"],
                 names=("out", "dx", "dW_gate_up", "dW_down", "d_topk_w"))


def test_persistent_recompute_equals_saved():
    """The backward that recomputes H and Aw through the persistent gate/up
    GEMM gives the saved path's gradients bit for bit."""
    wl = TINY.scaled(T=1500, d=384, E=16, k=4, I=320, **BF)
    inp = S.make_inputs(wl, seed=34)
    print("persistent case recompute", flush=True)
    _bit_equal(_run(wl, inp, True, save=False), _run(wl, inp, False),
               names=("out", "dx", "dW_gate_up", "dW_down", "d_topk_w", "dlogits"))


@pytest.mark.parametrize("name", ["q30b", "q235b"])
def test_persistent_full_size_bit_equal(name):
    """Full sizes, where every tile runs 32 (q30b) or 64 (q235b) K steps and
    the expert loads are uneven (q235b's routing bias)."""
    wl = S.WORKLOADS[name]
    inp = S.make_inputs(wl, seed=35)
    print(f"persistent case {name}", flush=True)
    a = _run(wl, inp, True)
    b = _run(wl, inp, False)
    _bit_equal(a, b)
    assert np.isfinite(to_np(a["out"])).all()
