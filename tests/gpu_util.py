"""Helpers shared by the GPU parity tests: run the HIP path through the C
ABI and the oracle on the same seeded inputs, and compare."""
import numpy as np
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
# (forward, backward) quantisation recipes of each fp8 precision
RECIPE = {"fp8_block": (O.FP8_BLOCK, O.FP8_BLOCK), "mxfp8": (O.MXFP8, O.MXFP8),
          "fp8_bwd": (O.NO_QUANT, O.FP8_BLOCK)}


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def to_np(t):
    return t.detach().cpu().double().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def run_gpu(wl, inp, ids=None, w=None, backward=True, limit=0.0):
    """Runs forward (+ backward) of the layer on cuda:0; returns CPU numpy
    results and the routing artefacts.  limit > 0: clamped SwiGLU."""
    dev = torch.device("cuda", 0)
    dt = S.torch_dtype(wl.dtype)
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=dt, logits_dtype=S.torch_dtype(wl.logits_dtype),
                       precision=wl.precision, device=dev, swiglu_limit=limit)
    x = inp["x"].to(dev)
    wgu = inp["w_gate_up"].to(dev)
    wd = inp["w_down"].to(dev)
    if ids is None:
        layer.forward(x, wgu, wd, logits=inp["logits"].to(dev))
    else:
        layer.forward(x, wgu, wd, topk_ids=ids.to(dev), topk_w=w.to(dev))
    res = {"out": to_np(layer.out)}
    r = layer.routing
    for n in ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of"):
        res[n] = to_np(getattr(r, n))
    if backward:
        g = layer.backward(inp["dout"].to(dev), x, wgu, wd)
        for n, v in g.items():
            res[n] = to_np(v)
    torch.cuda.synchronize()
    return res


def run_oracle(wl, inp, ids=None, w=None, backward=True, limit=0.0):
    f = lambda t: t.double().numpy()
    logits = f(inp["logits"]) if ids is None else None
    if ids is None:
        rt = O.route(logits, wl.k, wl.E)
    else:
        rt = O.route(None, wl.k, wl.E, ids=ids.numpy(), w=w.double().numpy())
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    recipes = RECIPE.get(wl.precision)
    if recipes is None:
        fw = O.forward(f(inp["x"]), rt, Wgu, Wd, limit=limit)
    else:
        fw = O.forward_fp8(f(inp["x"]), rt, Wgu, Wd, recipe=recipes[0], limit=limit)
    res = {"rt": rt, "out": fw["out"]}
    if backward:
        if recipes is None:
            bw = O.backward(f(inp["dout"]), rt, Wgu, Wd, fw, logits=logits, limit=limit)
        else:
            bw = O.backward_fp8(f(inp["dout"]), rt, Wgu, Wd, fw, logits=logits, recipe=recipes[1],
                                limit=limit)
        res.update(bw)
    return res


def bf16_test_matrix(shape, seed):
    """bf16 values spanning e4m3's normal and subnormal ranges after
    scaling: per-row magnitudes from 1e-6 to 1e3, a zero block, exact ties,
    and blocks whose largest magnitude is about 1e-37, so that their
    blockwise scale (amax / 448) lies below 2^-128 and has no finite float32
    reciprocal: the 128 x 128 block of rows 0..127 and columns 256..383 of
    the flattened matrix (a weight block, or 1 x 128 row blocks), with zeros
    in it, and column 130 (every 128-token run of it).  Blocks around 1e-31
    have a finite reciprocal scale but values below 2^-100, where one FMA
    correction of v / s is not exact and the quantisers divide, with nonzero
    codes: row 2, column 132 (its token runs) and, for weights, the block of
    rows 128..255, columns 0..127.  Column 131 spans 1e-38..1e-28 inside
    ordinary blocks, across that 2^-100 boundary."""
    g = np.random.default_rng(seed)
    a = g.standard_normal(shape) * np.exp(g.uniform(np.log(1e-6), np.log(1e3), shape[:-1] + (1,)))
    flat = a.reshape(-1, a.shape[-1])
    if flat.shape[0] >= 128 and flat.shape[1] >= 384:
        tiny = g.standard_normal((128, 128)) * 1e-37
        tiny[::7, 3] = 0.0
        flat[:128, 256:384] = tiny
    if flat.shape[0] >= 256 and flat.shape[1] >= 128:
        flat[128:256, :128] = g.standard_normal((128, 128)) * 1e-31
    if flat.shape[1] > 132:
        flat[:, 130] = g.standard_normal(flat.shape[0]) * 1e-37
        flat[::5, 130] = 0.0
        flat[:, 131] = g.standard_normal(flat.shape[0]) * 10.0 ** g.uniform(-38, -28, flat.shape[0])
        flat[:, 132] = g.standard_normal(flat.shape[0]) * 1e-31
    if flat.shape[0] > 2:
        flat[2] = g.standard_normal(flat.shape[1]) * 1e-31
    a = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    flat = a.view(-1, a.shape[-1])
    flat[0, :128] = 0.0                         # an all-zero block
    flat[1, :4] = torch.tensor([448.0, 224.0, 0.5, -0.5])
    return a.contiguous()


def check_routing(gpu, ref):
    rt = ref["rt"]
    assert np.array_equal(gpu["topk_ids"], rt["ids"]), "topk_ids"
    assert np.array_equal(gpu["counts"], rt["counts"]), "counts"
    assert np.array_equal(gpu["offsets"], rt["offsets"]), "offsets"
    assert np.array_equal(gpu["src_of"], rt["src_of"]), "src_of"
    assert np.array_equal(gpu["row_of"], rt["row_of"]), "row_of"
    assert rel_err(gpu["topk_w"], rt["w"]) < 1e-5, "topk_w"


def check_floats(gpu, ref, tol, names=("out", "dx", "dW_gate_up", "dW_down", "d_topk_w", "dlogits")):
    errs = {}
    for n in names:
        if n in gpu and n in ref:
            errs[n] = rel_err(gpu[n], ref[n])
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"tolerance {tol} exceeded: {bad} (all: {errs})"
    return errs
