"""Parity on seeded random layer shapes: every storage dtype and precision,
the clamped SwiGLU and the persistent engine, with extents drawn anywhere
the boundary allows them at test-friendly sizes (d, I multiples of 8, or of
128 for fp8; ragged expert loads; k up to E).  Clamped cases use the grid
inputs of the clamped-SwiGLU tests, so that both sides clamp the same
elements.  Each case is checked like the
fixed ones: routing bit-exact, floats within the layer tolerance, and the
persistent engine bit-equal to the default one."""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

from gpu_util import TOL, check_floats, check_routing, run_oracle, to_np
from test_gpu_clamped_swiglu import LIMIT, grid_inputs

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw(i):
    g = np.random.default_rng(1000 + i)
    prec = ["native", "native", "fp8_block", "mxfp8", "fp8_bwd"][i % 5]
    dtype = "f32" if prec == "native" and g.random() < 0.3 else "bf16"
    step = 128 if prec != "native" else 8
    d = int(step * g.integers(1, 513 // step + 1))
    I = int(step * g.integers(1, 513 // step + 1))
    E = int(g.integers(1, 49))
    k = int(min(E, g.integers(1, 9) if g.random() < 0.85 else g.integers(1, E + 1)))
    T = int(g.integers(1, 1501))
    lim = float(g.choice([0.0, 0.0, LIMIT]))
    persistent = bool(dtype == "bf16" and prec in ("native", "fp8_bwd") and g.random() < 0.4)
    wl = S.WORKLOADS["tiny"].scaled(T=T, d=d, E=E, k=k, I=I, dtype=dtype, logits_dtype=dtype, precision=prec)
    return wl, lim, persistent


def _run(wl, inp, lim, persistent):
    dev = torch.device("cuda", 0)
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=S.torch_dtype(wl.dtype),
                       logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=dev,
                       swiglu_limit=lim, persistent=persistent)
    x, wgu, wd = (inp[n].to(dev) for n in ("x", "w_gate_up", "w_down"))
    res = {"out": layer.forward(x, wgu, wd, logits=inp["logits"].to(dev)).clone()}
    for n in ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of"):
        res[n] = getattr(layer.routing, n).clone()
    res.update({n: v.clone() for n, v in layer.backward(inp["dout"].to(dev), x, wgu, wd).items()})
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    wl, lim, persistent = draw(i)
    print(f"case random {i}: {wl} limit={lim} persistent={persistent}", flush=True)
    # clamped cases take the clamped test's grid inputs, on which no
    # pre-activation lies near the limit
    inp = grid_inputs(wl, 2000 + i) if lim else S.make_inputs(wl, seed=2000 + i)
    got = _run(wl, inp, lim, persistent)
    if persistent:
        ref_gpu = _run(wl, inp, lim, False)
        for n in got:
            assert torch.equal(got[n], ref_gpu[n]), n
    ref = run_oracle(wl, inp, limit=lim)
    gnp = {n: to_np(v) for n, v in got.items()}
    check_routing(gnp, ref)
    tol = TOL["fp8"] if wl.precision != "native" else TOL[wl.dtype]
    errs = check_floats(gnp, ref, tol)
    print(i, errs)
