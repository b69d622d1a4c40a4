"""The layer's calls allocate nothing and never synchronise, so a caller
can capture forward + backward into one HIP graph (torch.cuda.CUDAGraph)
and replay it.  Every replay, with eager work on the same buffers in
between, must give the eager results bit for bit, in bf16 and in every fp8
precision, with the routing computed inside the graph."""
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16", logits_dtype="bf16")
CASES = {
    "bf16": S.WORKLOADS["tiny"].scaled(T=1500, d=384, E=16, k=4, I=320, **BF),
    "fp8_block": S.WORKLOADS["tiny"].scaled(T=900, d=256, E=8, k=2, I=256, precision="fp8_block", **BF),
    "mxfp8": S.WORKLOADS["tiny"].scaled(T=900, d=384, E=8, k=2, I=256, precision="mxfp8", **BF),
    "fp8_bwd": S.WORKLOADS["tiny"].scaled(T=700, d=256, E=12, k=3, I=384, precision="fp8_bwd", **BF),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_equal_eager(case):
    wl = CASES[case]
    print(f"graph case {case}", flush=True)
    dev = torch.device("cuda", 0)
    g = {n: t.to(dev) for n, t in S.make_inputs(wl, seed=41).items()}
    layer = B.MoeLayer(wl.T, wl.d, wl.E, wl.k, wl.I, dtype=S.torch_dtype(wl.dtype),
                       logits_dtype=S.torch_dtype(wl.logits_dtype), precision=wl.precision, device=dev)
    grads = {}

    def step():
        layer.forward(g["x"], g["w_gate_up"], g["w_down"], logits=g["logits"])
        grads.update(layer.backward(g["dout"], g["x"], g["w_gate_up"], g["w_down"]))

    step()
    torch.cuda.synchronize()
    ref = {"out": layer.out.clone(), "topk_ids": layer.routing.topk_ids.clone(),
           **{n: v.clone() for n, v in grads.items()}}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in list(grads.values()) + [layer.out]:
            t.fill_(float("nan"))          # eager work on the same buffers between replays
        layer.routing.topk_ids.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"out": layer.out, "topk_ids": layer.routing.topk_ids, **grads}
        for n, v in ref.items():
            assert torch.equal(got[n], v), (case, rep, n)
