"""Clamped SwiGLU layer (limit as an argument of the C ABI) against the
oracle, in every storage dtype and precision.

The clamp makes the SwiGLU's derivative jump at the limit, so a
pre-activation that the GPU and the oracle round to opposite sides of it
would differ by a finite amount.  The inputs are therefore on a coarse
dyadic grid: x in {0, +-0.5, +-1}, weights in {0, +-1/8} (+-1/16 for the
down weights), so that every gate/up pre-activation is a multiple of 1/16
that float32 sums exactly and bfloat16 stores exactly, and the limit sits
halfway between two grid points.  Both sides then clamp the same elements,
and the tolerances are the layer's own (1e-4 float32, 2e-2 bf16, 6e-2 fp8).
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import synthetic as S

from gpu_util import TOL, check_floats, check_routing, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

LIMIT = 1.03125          # 33/32: halfway between the grid points 1 and 1 + 1/16
TINY = S.WORKLOADS["tiny"]
BF = dict(dtype="bf16", logits_dtype="bf16")

CASES = {
    "f32": TINY,
    "bf16_tiles": TINY.scaled(T=777, d=384, E=16, k=4, I=320, **BF),
    "bf16_ktail": TINY.scaled(T=500, d=200, E=8, k=2, I=72, **BF),
    "fp8_block": TINY.scaled(T=600, d=256, E=8, k=2, I=256, precision="fp8_block", **BF),
    "mxfp8": TINY.scaled(T=600, d=256, E=8, k=2, I=256, precision="mxfp8", **BF),
    "fp8_bwd": TINY.scaled(T=600, d=256, E=8, k=2, I=256, precision="fp8_bwd", **BF),
    "q30b_t4096": S.WORKLOADS["q30b_t4096"],
}


def grid_inputs(wl, seed):
    """The workload's logits and dout, with x and both weights on the grid."""
    inp = S.make_inputs(wl, seed=seed)
    g = np.random.default_rng(seed)
    dt = S.torch_dtype(wl.dtype)
    inp["x"] = torch.from_numpy(g.choice([-1.0, -0.5, 0.0, 0.5, 1.0], (wl.T, wl.d)).astype(np.float32)).to(dt)
    inp["w_gate_up"] = torch.from_numpy(
        g.choice([-0.125, 0.0, 0.125], (wl.E, 2 * wl.I, wl.d)).astype(np.float32)).to(dt)
    inp["w_down"] = torch.from_numpy(
        g.choice([-0.0625, 0.0, 0.0625], (wl.E, wl.d, wl.I)).astype(np.float32)).to(dt)
    return inp


@pytest.mark.parametrize("name", list(CASES))
def test_clamped_swiglu_layer_parity(name):
    wl = CASES[name]
    print(f"case clamped {name}: {wl} limit={LIMIT}", flush=True)
    inp = grid_inputs(wl, seed=3)
    ref = run_oracle(wl, inp, limit=LIMIT)
    H = inp["x"].double().numpy() @ inp["w_gate_up"][0].double().numpy().T
    assert np.all(np.abs(np.abs(H) - LIMIT) >= 1 / 32)               # no value at the limit
    assert (H[:, :wl.I] > LIMIT).mean() > 0.02 and (np.abs(H[:, wl.I:]) > LIMIT).mean() > 0.05
    gpu = run_gpu(wl, inp, limit=LIMIT)
    check_routing(gpu, ref)
    tol = TOL["fp8"] if wl.precision != "native" else TOL[wl.dtype]
    errs = check_floats(gpu, ref, tol)
    if wl.precision == "fp8_bwd":
        assert errs["out"] <= TOL["bf16"]
    print(name, errs)


@pytest.mark.parametrize("name", ["bf16_tiles", "fp8_block"])
def test_clamped_recompute_and_operators_equal_saved_direct_calls(name):
    """The recomputing backward and the torch operators (moe_layer with
    swiglu_limit) run the same kernels with the clamp: bit-equal results."""
    from combine_top_route_amd import binding as B
    from combine_top_route_amd.autograd import moe_layer
    wl = CASES[name]
    print(f"case clamped operators {name}", flush=True)
    dev = torch.device("cuda", 0)
    inp = grid_inputs(wl, seed=4)
    x, lg, wgu, wd, dout = (inp[n].to(dev) for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    res = []
    for save in (True, False):
        layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=x.dtype, logits_dtype=lg.dtype,
                           precision=wl.precision, device=dev, save=save, swiglu_limit=LIMIT)
        out = layer.forward(x, wgu, wd, logits=lg).clone()
        g = layer.backward(dout, x, wgu, wd)
        res.append([out] + [g[n].clone() for n in ("dx", "dlogits", "dW_gate_up", "dW_down")])
    xg, lgg, wgug, wdg = (t.clone().requires_grad_() for t in (x, lg, wgu, wd))
    out = moe_layer(xg, lgg, wgug, wdg, wl.k, wl.precision, recompute=True, swiglu_limit=LIMIT)
    grads = torch.autograd.grad(out, (xg, lgg, wgug, wdg), dout)
    res.append([out.detach()] + list(grads))
    torch.cuda.synchronize()
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert torch.equal(a, b)
    # and the clamp is really in effect: the plain layer differs
    plain = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=x.dtype, logits_dtype=lg.dtype,
                       precision=wl.precision, device=dev)
    assert not torch.equal(plain.forward(x, wgu, wd, logits=lg), res[0][0])


@pytest.mark.parametrize("name", ["bf16_tiles", "bf16_ktail", "fp8_bwd"])
def test_clamped_persistent_equals_default_and_oracle(name):
    """The persistent row GEMMs (MOE_FLAG_PERSISTENT) apply the clamp in
    their own gate/up epilogue: results bit-equal to the default engine's
    and within the layer tolerance of the oracle."""
    from combine_top_route_amd import binding as B
    wl = CASES[name]
    print(f"case clamped persistent {name}: {wl} limit={LIMIT}", flush=True)
    inp = grid_inputs(wl, seed=5)
    dev = torch.device("cuda", 0)
    x, wgu, wd, lg, dout = (inp[n].to(dev) for n in ("x", "w_gate_up", "w_down", "logits", "dout"))
    res = []
    for persistent in (True, False):
        layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=S.torch_dtype(wl.dtype),
                           logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=dev,
                           swiglu_limit=LIMIT, persistent=persistent)
        out = layer.forward(x, wgu, wd, logits=lg).clone()
        g = {n: v.clone() for n, v in layer.backward(dout, x, wgu, wd).items()}
        torch.cuda.synchronize()
        res.append({"out": out, "saved": layer.saved.clone(), **g})
    for n in res[1]:
        assert torch.equal(res[0][n], res[1][n]), n
    ref = run_oracle(wl, inp, limit=LIMIT)
    got = {n: v.cpu().double().numpy() for n, v in res[0].items() if n != "saved"}
    tol = TOL["fp8"] if wl.precision != "native" else TOL[wl.dtype]
    check_floats(got, ref, tol)
