"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Integer routing artefacts must match bit for bit; floating outputs and
gradients within max|err|/max|ref| <= 1e-4 (float32 storage), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O

from gpu_util import TOL, check_floats, check_routing, rel_err, run_gpu, run_oracle, to_np

pytestmark = pytest.mark.gpu

TINY = S.WORKLOADS["tiny"]
BF = dict(dtype="bf16", logits_dtype="bf16")

SMALL_CASES = {
    # float32 storage (plain FMA path)
    "tiny": TINY,
    "f32_ragged": TINY.scaled(T=100, d=48, E=5, k=3, I=40),
    # bf16 MFMA path: several tiles, ragged row tails, N and K tails
    "bf16_tiles": TINY.scaled(T=777, d=384, E=16, k=4, I=320, **BF),
    "bf16_ktail": TINY.scaled(T=1000, d=200, E=16, k=4, I=72, **BF),
    "bf16_bigrows": TINY.scaled(T=2048, d=256, E=4, k=2, I=192, **BF),
    "bf16_one_token": TINY.scaled(T=1, d=128, E=8, k=2, I=64, **BF),
    "bf16_k_equals_E": TINY.scaled(T=64, d=128, E=4, k=4, I=64, **BF),
    "bf16_single_expert": TINY.scaled(T=200, d=128, E=1, k=1, I=128, **BF),
    "bf16_k80": TINY.scaled(T=16, d=64, E=128, k=80, I=64, **BF),
    "bf16_k12": TINY.scaled(T=200, d=128, E=32, k=12, I=64, **BF),
    "bf16_k20": TINY.scaled(T=100, d=128, E=64, k=20, I=64, **BF),
    # 12 experts: two weight-gradient slots per XCD, four of the 16 empty
    "bf16_e12": TINY.scaled(T=300, d=128, E=12, k=3, I=64, **BF),
    "bf16_d4096": TINY.scaled(T=64, d=4096, E=8, k=2, I=256, **BF),
    "bf16_f32_logits": TINY.scaled(T=300, d=256, E=16, k=4, I=128, dtype="bf16", logits_dtype="f32"),
    # the smallest and largest extents the boundary accepts (d, I multiples
    # of 8 in [8, 16384]): one-step K loops with an 8-wide tail, 8-column N
    # tiles, and 256-step K loops
    "bf16_min_dims": TINY.scaled(T=333, d=8, E=6, k=2, I=8, **BF),
    "f32_min_dims": TINY.scaled(T=333, d=8, E=6, k=2, I=8),
    "bf16_max_d": TINY.scaled(T=40, d=16384, E=4, k=2, I=64, **BF),
    "bf16_max_i": TINY.scaled(T=40, d=64, E=3, k=2, I=16384, **BF),
    # intermediate size above the hidden size (the backward's I-wide
    # intermediates must not fit a d-wide buffer by accident)
    "bf16_wide_i": TINY.scaled(T=500, d=136, E=8, k=2, I=648, **BF),
    # the most experts the boundary accepts: about a dozen rows each, many
    # experts empty, every row tile a quarter-height tail
    "bf16_e1024": TINY.scaled(T=1500, d=64, E=1024, k=8, I=64, **BF),
    # few experts with many rows (token operands larger than the weights):
    # every row GEMM takes its tiles row-tile-major, ragged row tiles and
    # two to four N tiles per expert
    "bf16_ep_share": TINY.scaled(T=3000, d=512, E=2, k=1, I=512, **BF),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_layer_parity_small(name):
    wl = SMALL_CASES[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=1)
    gpu = run_gpu(wl, inp)
    ref = run_oracle(wl, inp)
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL[wl.dtype])
    print(name, errs)


def test_layer_parity_ids_in_with_empty_and_hot_experts():
    wl = TINY.scaled(T=1500, d=256, E=16, k=4, I=128, **BF)
    ids, w = S.random_topk(wl.T, wl.E - 3, wl.k, seed=5)
    ids = ids + (ids >= 2).int() + (ids >= 5).int() + (ids >= 11).int()   # experts 2, 6, 13 ... get none
    ids = ids.numpy()
    ids[:1000, 0] = np.where((ids[:1000, 1:] == 0).any(1), ids[:1000, 0], 0)  # expert 0 is hot
    ids = torch.from_numpy(np.ascontiguousarray(ids.astype(np.int32)))
    inp = S.make_inputs(wl, seed=2)
    gpu = run_gpu(wl, inp, ids=ids, w=w)
    ref = run_oracle(wl, inp, ids=ids, w=w)
    assert (ref["rt"]["counts"] == 0).sum() >= 3 and ref["rt"]["counts"].max() > 900
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL["bf16"], names=("out", "dx", "dW_gate_up", "dW_down", "d_topk_w"))
    for e in np.nonzero(ref["rt"]["counts"] == 0)[0]:
        assert np.all(gpu["dW_gate_up"][e] == 0) and np.all(gpu["dW_down"][e] == 0)
    print(errs)


def test_layer_parity_q30b_t4096():
    """Qwen3-30B-A3B layer shape at 4096 tokens, every element."""
    wl = S.WORKLOADS["q30b_t4096"]
    inp = S.make_inputs(wl, seed=0)
    gpu = run_gpu(wl, inp)
    ref = run_oracle(wl, inp)
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL["bf16"])
    print(errs)


@pytest.mark.parametrize("name", ["q30b", "q235b", "q30b_ep8"])
def test_layer_parity_full_size_sampled(name):
    """Qwen3-30B-A3B and Qwen3-235B-A22B layer shapes at 16,384 tokens, and
    one GPU's share of the former under 8-way expert parallelism (16
    experts, 131,072 single-row tokens), in the benchmark's launch
    configuration: all routing artefacts bit-exact; out, dx, top-k-weight and
    logit gradients on sampled tokens; weight gradients of expert 0, of the
    busiest expert (q235b's router bias gives it about five times the mean
    load) and, for q235b, of a median one."""
    wl = S.WORKLOADS[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=0)
    gpu = run_gpu(wl, inp)
    lg = inp["logits"].double().numpy()
    rt = O.route(lg, wl.k, wl.E)
    check_routing(gpu, {"rt": rt})
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    x, dout = inp["x"].double().numpy(), inp["dout"].double().numpy()
    toks = np.random.default_rng(0).choice(wl.T, 24, replace=False)
    toks[:2] = [0, wl.T - 1]
    s = O.forward_backward_tokens(x, lg, dout, Wgu, Wd, wl.k, toks)
    for n in ("out", "dx", "d_topk_w", "dlogits"):
        e = rel_err(gpu[n][toks], s[n])
        assert e <= TOL["bf16"], (n, e)
    c = rt["counts"]
    experts = [0, int(np.argmax(c))]
    if name == "q235b":
        assert c.max() >= 4 * c.mean()
        experts.append(int(np.argsort(c)[len(c) // 2]))
    for e in experts:
        dgu, dd = O.expert_weight_grads(x, dout, rt, Wgu, Wd, e)
        for n, got, ref in (("dW_gate_up", gpu["dW_gate_up"][e], dgu), ("dW_down", gpu["dW_down"][e], dd)):
            err = rel_err(got, ref)
            print(n, e, c[e], err)
            assert err <= TOL["bf16"], (n, e, err)


def test_deterministic_bitwise():
    wl = TINY.scaled(T=1024, d=256, E=16, k=4, I=192, **BF)
    inp = S.make_inputs(wl, seed=3)
    a = run_gpu(wl, inp)
    b = run_gpu(wl, inp)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_permute_combine_identity(dtype):
    """Identity experts: dispatch then combine returns the input (k=1, w=1:
    bit for bit; renormalised top-k weights: to within one rounding)."""
    dev = torch.device("cuda", 0)
    wl = TINY.scaled(T=515, d=136, E=8, k=1, dtype=dtype, logits_dtype=dtype)
    inp = S.make_inputs(wl, seed=4)
    x = inp["x"].to(dev)
    ids, _ = S.random_topk(wl.T, wl.E, 1, seed=4)
    r = B.route_ids(ids.to(dev), torch.ones((wl.T, 1), dtype=torch.float32, device=dev), wl.E)
    xp = B.permute(x, r, 1)
    out = B.combine(xp, r, wl.T, 1)
    assert torch.equal(out, x)
    rt = O.route(None, 1, wl.E, ids=ids.numpy(), w=np.ones((wl.T, 1)))
    assert np.array_equal(to_np(xp), O.dispatch(inp["x"].double().numpy(), rt))
    wl4 = wl.scaled(k=4)
    r4 = B.route(inp["logits"].to(dev)[:, :8].contiguous(), 4)
    xp4 = B.permute(x, r4, 4)
    out4 = B.combine(xp4, r4, wl.T, 4)
    ref = inp["x"].double().numpy()
    ulp = 2.0 ** -23 if dtype == "f32" else 2.0 ** -8
    assert np.max(np.abs(to_np(out4) - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2 * ulp


@pytest.mark.parametrize("ldt", ["f32", "bf16"])
@pytest.mark.parametrize("E,k", [(16, 2), (128, 8), (12, 5), (40, 12), (64, 20), (128, 80),
                                 (1024, 8), (1000, 16), (1024, 100), (1024, 1024), (2, 1), (2, 2)])
def test_routing_signed_zeros_and_minus_inf(ldt, E, k):
    """Logits with +0.0 / -0.0 ties at the selection boundary and -inf
    entries, including rows with fewer than k finite logits (their -inf
    experts are selected lowest index first, with weight exactly 0): ids,
    counts, offsets and the permutation bit-exact against the oracle, on
    every top-k kernel (k <= 8, <= 16 with and without the four-lane split,
    <= 64, and above)."""
    dev = torch.device("cuda", 0)
    T = 301
    g = np.random.default_rng(E * 1000 + k)
    lg = np.round(g.standard_normal((T, E)))          # small integers: ties everywhere
    lg[g.random((T, E)) < 0.3] = 0.0
    neg = g.random((T, E)) < 0.5
    lg[(lg == 0) & neg] = -0.0                        # signed zeros tie with +0.0
    lg[g.random((T, E)) < 0.1] = -np.inf
    for t in range(0, T, 5):                          # rows with 1..k finite logits
        nfin = int(g.integers(1, k + 1))
        row = np.full(E, -np.inf)
        keep = g.choice(E, nfin, replace=False)
        row[keep] = np.round(g.standard_normal(nfin))
        lg[t] = row
    lg[1] = 0.0
    lg[1, ::2] = -0.0                                 # a row of zeros only
    lg[:, 0][np.isinf(lg).all(axis=1)] = 0.0          # at least one finite logit per row
    assert np.signbit(lg[lg == 0]).any() and np.isinf(lg).any()
    logits = torch.from_numpy(lg.astype(np.float32)).to(S.torch_dtype(ldt))
    assert np.array_equal(logits.double().numpy(), lg)
    r = B.route(logits.to(dev), k)
    torch.cuda.synchronize()
    rt = O.route(lg, k, E)
    check_routing({n: to_np(getattr(r, n)) for n in ("topk_ids", "topk_w", "counts", "offsets",
                                                      "row_of", "src_of")}, {"rt": rt})
    w = to_np(r.topk_w)
    sel = np.take_along_axis(lg, rt["ids"], axis=1)
    assert np.all(w[np.isinf(sel)] == 0.0) and np.all(w[~np.isinf(sel)] > 0.0)


@pytest.mark.parametrize("T,d,E,k", [(4096, 2048, 128, 8), (1000, 4096, 64, 6), (300, 256, 16, 4)])
def test_permute_bit_exact(T, d, E, k):
    """moe_permute (dispatch alone) against the oracle's dispatch, every
    element: rows of 4 and 8 KB take the token scatter (each token's row
    written to its k expert-sorted rows), other widths the row gather."""
    dev = torch.device("cuda", 0)
    print(f"case permute T={T} d={d} E={E} k={k}", flush=True)
    wl = S.WORKLOADS["q30b"].scaled(T=T, d=d, E=E, k=k)
    logits = S.make_logits(wl, seed=7)
    g = np.random.default_rng(7)
    x = torch.from_numpy(g.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    r = B.route(logits.to(dev), k)
    xp = B.permute(x.to(dev), r, k)
    torch.cuda.synchronize()
    rt = O.route(logits.double().numpy(), k, E)
    assert np.array_equal(to_np(r.src_of), rt["src_of"])
    assert np.array_equal(to_np(xp), O.dispatch(x.double().numpy(), rt))
