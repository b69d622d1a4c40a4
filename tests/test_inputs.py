"""Realised statistics of the synthetic workloads (CPU only).

The skewed workload must give the hottest expert about 10x the mean load and
at least 4 empty experts; the Qwen3-30B-shaped workload must be near-uniform.
Routing here is the oracle's.
"""
import numpy as np
import pytest

from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O


def _counts(name, seed=0, T=None):
    wl = S.WORKLOADS[name]
    lg = S.make_logits(wl, seed=seed, T=T).double().numpy()
    ids = O.topk_select(lg, wl.k)
    return O.expert_counts_fast(ids, wl.E)[0]


def test_near_uniform_load_q30b():
    c = _counts("q30b")
    assert c.sum() == 16384 * 8
    assert c.max() / c.mean() < 1.2 and c.min() / c.mean() > 0.8


@pytest.mark.parametrize("seed", [0, 1])
def test_skewed_load_fp8(seed):
    c = _counts("fp8_skew", seed)
    assert 9.0 < c.max() / c.mean() < 11.0
    assert (c == 0).sum() >= 4


def test_mild_imbalance_q235b():
    c = _counts("q235b")
    assert 2.0 < c.max() / c.mean() < 8.0
    assert (c == 0).sum() == 0


def test_generators_are_seeded_and_thread_independent():
    wl = S.WORKLOADS["tiny"]
    a = S.make_inputs(wl, seed=3, threads=1)
    b = S.make_inputs(wl, seed=3, threads=4)
    c = S.make_inputs(wl, seed=4, threads=4)
    for k in a:
        assert a[k].equal(b[k])
        assert not a[k].equal(c[k])
    x = a["x"].double().numpy()
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    w = a["w_gate_up"].double().numpy()
    assert abs(w.std() * np.sqrt(wl.d) - 1) < 0.05
