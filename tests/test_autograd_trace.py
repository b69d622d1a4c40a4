"""The layer's torch operators trace without a GPU: their fake (shape-only)
implementations give the right output shapes and dtypes, and forward plus
backward trace into one graph under fake tensors.  CPU only; the library is
loaded for its host-side size queries."""
import os

import pytest
import torch

from combine_top_route_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")

T, d, E, k, I = 64, 256, 8, 2, 128


def _inputs(device, dtype=torch.bfloat16):
    return (torch.empty(T, d, dtype=dtype, device=device), torch.empty(T, E, dtype=dtype, device=device),
            torch.empty(E, 2 * I, d, dtype=dtype, device=device), torch.empty(E, d, I, dtype=dtype, device=device))


@pytest.mark.parametrize("precision,save", [("native", True), ("native", False), ("fp8_block", True),
                                            ("mxfp8", True)])
def test_fake_shapes(precision, save):
    from combine_top_route_amd import autograd  # noqa: F401  (registers the operators)
    x, lg, wgu, wd = _inputs("meta")
    outs = torch.ops.ctr_moe.moe_fwd(x, lg, wgu, wd, k, precision, save)
    shape = B.make_shape(T, d, E, k, I, torch.bfloat16, torch.bfloat16, precision)
    want = [((T, d), torch.bfloat16), ((B.saved_size(shape) if save else 0,), torch.uint8),
            ((T, k), torch.int32), ((T, k), torch.float32), ((E,), torch.int32), ((E + 1,), torch.int32),
            ((T * k,), torch.int32), ((T * k,), torch.int32)]
    assert [(tuple(o.shape), o.dtype) for o in outs] == want
    g = torch.ops.ctr_moe.moe_bwd(torch.empty(T, d, dtype=torch.bfloat16, device="meta"), x, lg, wgu, wd,
                                  *outs[1:], k, precision)
    assert [tuple(t.shape) for t in g] == [(T, d), (T, E), (E, 2 * I, d), (E, d, I)]


def test_forward_and_backward_trace_into_one_graph():
    from torch.fx.experimental.proxy_tensor import make_fx

    from combine_top_route_amd.autograd import moe_layer

    def step(x, lg, wgu, wd, dout):
        out = moe_layer(x, lg, wgu, wd, k, recompute=True)
        return torch.autograd.grad(out, (x, lg, wgu, wd), dout)

    x, lg, wgu, wd = (t.requires_grad_() for t in _inputs("cpu"))
    dout = torch.empty(T, d, dtype=torch.bfloat16)
    gm = make_fx(step, tracing_mode="fake")(x, lg, wgu, wd, dout)
    targets = [str(n.target) for n in gm.graph.nodes if n.op == "call_function"]
    assert any("ctr_moe.moe_fwd" in t for t in targets)
    assert any("ctr_moe.moe_bwd" in t for t in targets)


@pytest.mark.parametrize("case", ["w_down_shape", "logits_shape", "x_d", "k_range", "dtype_mix",
                                  "not_contiguous", "cpu_tensors", "precision"])
def test_operators_reject_bad_arguments_before_any_launch(case):
    """The real (non-fake) operator implementations validate shapes, dtypes,
    contiguity and device and raise ValueError before the C ABI is called;
    here every case runs on the CPU, where a launch could not happen."""
    from combine_top_route_amd import autograd  # noqa: F401
    x, lg, wgu, wd = _inputs("cpu")
    kk, prec = k, "native"
    if case == "w_down_shape":
        wd = torch.empty(E, d, I + 8, dtype=torch.bfloat16)
    elif case == "logits_shape":
        lg = torch.empty(T, E + 1, dtype=torch.bfloat16)
    elif case == "x_d":
        x = torch.empty(T, d + 8, dtype=torch.bfloat16)
    elif case == "k_range":
        kk = E + 1
    elif case == "dtype_mix":
        wd = wd.float()
    elif case == "not_contiguous":
        x = torch.empty(d, T, dtype=torch.bfloat16).t()
    elif case == "precision":
        prec = "fp4"
    match = "one GPU" if case == "cpu_tensors" else "must be|outside|unknown|dtype"
    with pytest.raises(ValueError, match=match):
        torch.ops.ctr_moe.moe_fwd(x, lg, wgu, wd, kk, prec, True)


def test_backward_operator_rejects_bad_routing_and_saved():
    from combine_top_route_amd import autograd  # noqa: F401
    x, lg, wgu, wd = _inputs("cpu")
    dout = torch.empty(T, d, dtype=torch.bfloat16)
    i32 = dict(dtype=torch.int32)
    good = [torch.empty(0, dtype=torch.uint8), torch.empty(T, k, **i32), torch.empty(T, k),
            torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32)]
    bad_cases = []
    for i, repl in ((1, torch.empty(T, k + 1, **i32)), (2, torch.empty(T, k, dtype=torch.float64)),
                    (5, torch.empty(T * k - 1, **i32)), (0, torch.empty(7, dtype=torch.uint8))):
        args = list(good)
        args[i] = repl
        bad_cases.append(args)
    for args, what in zip(bad_cases, ("topk_ids", "topk_w", "row_of", "saved holds")):
        with pytest.raises(ValueError, match=what):
            torch.ops.ctr_moe.moe_bwd(dout, x, lg, wgu, wd, *args, k, "native")
    with pytest.raises(ValueError, match="dout"):   # dout of the wrong shape
        torch.ops.ctr_moe.moe_bwd(torch.empty(T, d + 8, dtype=torch.bfloat16), x, lg, wgu, wd, *good, k, "native")
    with pytest.raises(ValueError, match="one GPU"):   # all well formed, but on the CPU
        torch.ops.ctr_moe.moe_bwd(dout, x, lg, wgu, wd, *good, k, "native")
