"""Every buffer the layer writes stays within its extent, reads leave the
inputs untouched, and results do not depend on what the workspaces, the
saved buffer or the outputs held before the call.

Each buffer handed to the C ABI sits between two 64 KiB guard bands of a
known byte; the outputs, workspaces and saved buffer start out filled with
0xFF (a NaN in every float format, -1 in int32).  After forward and backward
the guard bands must be intact, the inputs bit-identical to their copies,
and every output bit-equal to a run on freshly allocated buffers.
"""
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
GUARD = 64 * 1024
BAND = 0xA5
TINY = S.WORKLOADS["tiny"]
BF = dict(dtype="bf16", logits_dtype="bf16")

CASES = {
    "f32": (TINY.scaled(T=200, d=48, E=5, k=3, I=88), {}),
    "bf16_wide_i": (TINY.scaled(T=300, d=136, E=8, k=2, I=648, **BF), {}),
    "bf16_wide_d": (TINY.scaled(T=300, d=520, E=8, k=3, I=72, **BF), {}),
    "bf16_empty_experts": (TINY.scaled(T=20, d=128, E=64, k=2, I=256, **BF), {}),
    "bf16_persistent": (TINY.scaled(T=300, d=136, E=8, k=2, I=648, **BF), dict(persistent=True)),
    "bf16_recompute": (TINY.scaled(T=300, d=136, E=8, k=2, I=648, **BF), dict(save=False)),
    "bf16_clamped": (TINY.scaled(T=300, d=256, E=8, k=2, I=384, **BF), dict(swiglu_limit=7.0)),
    "fp8_block_wide_i": (TINY.scaled(T=300, d=256, E=8, k=2, I=640, precision="fp8_block", **BF), {}),
    "fp8_block_recompute": (TINY.scaled(T=300, d=256, E=8, k=2, I=640, precision="fp8_block", **BF),
                            dict(save=False)),
    "mxfp8_wide_d": (TINY.scaled(T=300, d=640, E=8, k=2, I=128, precision="mxfp8", **BF), {}),
    "fp8_bwd_wide_i": (TINY.scaled(T=300, d=128, E=8, k=2, I=384, precision="fp8_bwd", **BF), {}),
}


class Guarded:
    """A device buffer of `nbytes` between two guard bands."""

    def __init__(self, nbytes, fill):
        self.n = nbytes
        self.raw = torch.full((2 * GUARD + nbytes,), BAND, dtype=torch.uint8, device=DEV)
        self.body = self.raw[GUARD:GUARD + nbytes]
        if fill is not None:
            self.body.fill_(fill)

    def view(self, dtype, shape):
        return self.body.view(dtype).view(shape)

    def bands_intact(self):
        return bool((self.raw[:GUARD] == BAND).all() and (self.raw[GUARD + self.n:] == BAND).all())


def _guard_like(t, fill=None):
    """A guarded copy of tensor t (fill None: its values)."""
    g = Guarded(t.numel() * t.element_size(), 0xFF if fill is None else fill)
    v = g.view(t.dtype, t.shape)
    if fill is None:
        v.copy_(t)
    return g, v


def _run(layer, x, wgu, wd, logits, dout):
    layer.forward(x, wgu, wd, logits=logits)
    g = layer.backward(dout, x, wgu, wd)
    torch.cuda.synchronize()
    res = {"out": layer.out.clone(), **{n: v.clone() for n, v in g.items()}}
    for n in ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of"):
        res[n] = getattr(layer.routing, n).clone()
    return res


def _bits(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("name", list(CASES))
def test_writes_stay_in_bounds_and_ignore_prior_contents(name):
    wl, opt = CASES[name]
    print(f"case {name}: {wl} {opt}", flush=True)
    dt, ldt = S.torch_dtype(wl.dtype), S.torch_dtype(wl.logits_dtype)
    inp = {n: t.to(DEV) for n, t in S.make_inputs(wl, seed=4).items()}
    kw = dict(dtype=dt, logits_dtype=ldt, precision=wl.precision, device=DEV, **opt)

    ref = _run(B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, **kw), inp["x"], inp["w_gate_up"],
               inp["w_down"], inp["logits"], inp["dout"])

    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, **kw)
    guards = {}
    # outputs, workspaces and the saved buffer: 0xFF inside the bands
    for n in ("ws_fwd", "ws_bwd", "saved", "out", "dx", "dw_gate_up", "dw_down", "d_topk_w", "dlogits"):
        t = getattr(layer, n)
        if t is None:
            continue
        guards[n], v = _guard_like(t, fill=0xFF)
        setattr(layer, n, v)
    r = layer.routing
    for n in ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of"):
        guards[n], v = _guard_like(getattr(r, n), fill=0xFF)
        setattr(r, n, v)
    # inputs: copied between bands, compared after the calls
    ins = {}
    for n in ("x", "w_gate_up", "w_down", "logits", "dout"):
        guards[n], ins[n] = _guard_like(inp[n])

    got = _run(layer, ins["x"], ins["w_gate_up"], ins["w_down"], ins["logits"], ins["dout"])

    broken = [n for n, g in guards.items() if not g.bands_intact()]
    assert not broken, f"writes outside the buffers: {broken}"
    for n in ins:
        assert torch.equal(_bits(ins[n]), _bits(inp[n])), f"input {n} was written"
    assert set(got) == set(ref)
    for n in ref:
        assert torch.equal(_bits(got[n]), _bits(ref[n])), f"{n} differs from a run on fresh buffers"
