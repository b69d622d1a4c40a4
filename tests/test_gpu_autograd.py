"""The torch operators and the recomputing backward on the GPU.

* the autograd path returns exactly what direct calls of the C ABI return
  (same kernels, same inputs: bit-equal);
* the recomputing backward (saved == NULL) equals the saved one bit for bit
  in every precision;
* torch.compile(fullgraph=True) runs forward and backward through the
  operators without graph breaks, with the eager results;
* one case against the oracle.
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S
from combine_top_route_amd.autograd import moe_layer

from gpu_util import TOL, check_floats, run_oracle, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
CASES = {
    "f32": S.WORKLOADS["tiny"],
    "bf16": S.WORKLOADS["tiny"].scaled(T=300, d=256, E=16, k=4, I=128, dtype="bf16", logits_dtype="bf16"),
    "fp8_block": S.WORKLOADS["tiny"].scaled(T=300, d=256, E=16, k=4, I=128, dtype="bf16",
                                            logits_dtype="bf16", precision="fp8_block"),
    "mxfp8": S.WORKLOADS["tiny"].scaled(T=300, d=256, E=16, k=4, I=128, dtype="bf16",
                                        logits_dtype="bf16", precision="mxfp8"),
    "fp8_bwd": S.WORKLOADS["tiny"].scaled(T=300, d=256, E=16, k=4, I=128, dtype="bf16",
                                          logits_dtype="bf16", precision="fp8_bwd"),
    # intermediate size five times the hidden size
    "bf16_wide_i": S.WORKLOADS["tiny"].scaled(T=300, d=128, E=8, k=2, I=640, dtype="bf16",
                                              logits_dtype="bf16"),
    "fp8_block_wide_i": S.WORKLOADS["tiny"].scaled(T=300, d=128, E=8, k=2, I=640, dtype="bf16",
                                                   logits_dtype="bf16", precision="fp8_block"),
}
GRADS = ("dx", "dlogits", "dW_gate_up", "dW_down")


def _direct(wl, inp, save):
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=S.torch_dtype(wl.dtype),
                       logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=DEV,
                       save=save)
    x, wgu, wd = (inp[n].to(DEV) for n in ("x", "w_gate_up", "w_down"))
    out = layer.forward(x, wgu, wd, logits=inp["logits"].to(DEV)).clone()
    g = layer.backward(inp["dout"].to(DEV), x, wgu, wd)
    torch.cuda.synchronize()
    return {"out": out.cpu(), **{n: g[n].cpu() for n in GRADS}}


def _autograd(wl, inp, recompute, fn=None):
    x, lg, wgu, wd = (inp[n].to(DEV).requires_grad_() for n in ("x", "logits", "w_gate_up", "w_down"))
    dout = inp["dout"].to(DEV)

    def step(x, lg, wgu, wd):
        out = moe_layer(x, lg, wgu, wd, wl.k, wl.precision, recompute)
        return out, torch.autograd.grad(out, (x, lg, wgu, wd), dout)
    out, g = (fn or step)(x, lg, wgu, wd)
    torch.cuda.synchronize()
    return {"out": out.detach().cpu(), **{n: t.cpu() for n, t in zip(GRADS, g)}}


def _equal(a, b):
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name", list(CASES))
def test_recompute_equals_saved_bitwise(name):
    wl = CASES[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=3)
    _equal(_direct(wl, inp, save=True), _direct(wl, inp, save=False))


@pytest.mark.parametrize("name", ["bf16", "mxfp8"])
@pytest.mark.parametrize("recompute", [False, True])
def test_autograd_equals_direct_calls(name, recompute):
    wl = CASES[name]
    print(f"case {name} recompute={recompute}", flush=True)
    inp = S.make_inputs(wl, seed=4)
    _equal(_direct(wl, inp, save=True), _autograd(wl, inp, recompute))


@pytest.mark.parametrize("backend", ["aot_eager", "inductor"])
def test_compile_fullgraph_matches_eager(backend):
    """The forward compiles as one graph (no breaks); AOT autograd traces the
    backward through the backward operator.  inductor is the default
    compiler: it generates the surrounding elementwise kernels and calls the
    layer's operators as they are."""
    wl = CASES["bf16"]
    inp = S.make_inputs(wl, seed=5)
    print(f"compile backend {backend}", flush=True)

    def fwd(x, lg, wgu, wd):
        return moe_layer(x, lg, wgu, wd, wl.k, "native", True) * 2.0
    torch._dynamo.reset()
    compiled = torch.compile(fwd, fullgraph=True, backend=backend)
    res = []
    for f in (fwd, compiled):
        x, lg, wgu, wd = (inp[n].to(DEV).requires_grad_() for n in ("x", "logits", "w_gate_up", "w_down"))
        out = f(x, lg, wgu, wd)
        g = torch.autograd.grad(out, (x, lg, wgu, wd), inp["dout"].to(DEV))
        torch.cuda.synchronize()
        res.append({"out": out.detach().cpu(), **{n: t.cpu() for n, t in zip(GRADS, g)}})
    _equal(res[0], res[1])


def test_autograd_against_oracle():
    wl = CASES["bf16"]
    inp = S.make_inputs(wl, seed=6)
    got = _autograd(wl, inp, recompute=True)
    ref = run_oracle(wl, inp)
    gpu = {"out": to_np(got["out"]), "dx": to_np(got["dx"]), "dlogits": to_np(got["dlogits"]),
           "dW_gate_up": to_np(got["dW_gate_up"]), "dW_down": to_np(got["dW_down"])}
    errs = check_floats(gpu, ref, TOL["bf16"])
    print(errs)
