"""moe_route_noalloc (routing with the library's own fixed scratch array, no
workspace) against moe_route with a caller workspace, through the C ABI:
identical routing artefacts, bit for bit, on two calls in a row, the second
smaller than the first (the array keeps the first call's contents), in both
routing forms."""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S

pytestmark = pytest.mark.gpu

NAMES = ("topk_ids", "topk_w", "counts", "offsets", "row_of", "src_of")


def _compare(a, b):
    for n in NAMES:
        x, y = getattr(a, n).cpu(), getattr(b, n).cpu()
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), n


def test_route_noalloc_equals_route_twice():
    dev = torch.device("cuda", 0)
    # the q30b routing shape, then a smaller and differently shaped one
    for T, E, k, seed in ((16384, 128, 8, 0), (1000, 40, 6, 1)):
        print(f"case noalloc logits T={T} E={E} k={k}", flush=True)
        wl = S.WORKLOADS["q30b"].scaled(T=T, E=E, k=k)
        logits = S.make_logits(wl, seed=seed).to(dev)
        ref = B.route(logits, k)
        got = B.Routing.empty(T, E, k, dev, logits=logits)
        B.route_noalloc(got, T, E, k, logits.dtype)
        torch.cuda.synchronize()
        _compare(got, ref)
        assert int(got.offsets[-1]) == T * k
    # ids-in form, after the two calls above
    T, E, k = 700, 24, 3
    print(f"case noalloc ids T={T} E={E} k={k}", flush=True)
    ids, w = S.random_topk(T, E, k, seed=5)
    ids, w = ids.to(dev), w.to(dev)
    ref = B.route_ids(ids, w, E)
    got = B.Routing.empty(T, E, k, dev, topk_ids=ids, topk_w=w)
    B.route_noalloc(got, T, E, k)
    torch.cuda.synchronize()
    _compare(got, ref)
