"""Blockwise fp8 (OCP e4m3, fp32 block scales) path against the oracle.

Quantisation is byte work and must match bit for bit: every e4m3 code and
every scale.  Layer outputs and gradients match the oracle's emulation of the
same quantisation within max|err|/max|ref| <= 6e-2.
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O

from gpu_util import TOL, bf16_test_matrix, check_floats, check_routing, rel_err, run_gpu, run_oracle, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
FP8 = dict(dtype="bf16", logits_dtype="bf16", precision="fp8_block")
BASE = S.WORKLOADS["tiny"].scaled(**FP8)


def _decode(q, s_expanded):
    return q.view(torch.float8_e4m3fn).double().cpu().numpy() * s_expanded


def test_quantize_rows_bit_exact():
    x = bf16_test_matrix((300, 512), 1)
    q, s = B.quantize_fp8(x.to(DEV), B.QUANT_ROWS)
    s_np = s.cpu().numpy().astype(np.float64)
    ref = O.quant_rows_1x128(x.float().numpy())
    got = _decode(q, np.repeat(s_np, 128, axis=1))
    assert np.array_equal(got, ref)
    # codes: the oracle's values over the (equal) scales, cast to e4m3
    codes = torch.from_numpy(ref / np.repeat(s_np, 128, axis=1)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(q.cpu(), codes)


@pytest.mark.parametrize("kind", [B.QUANT_WEIGHT, B.QUANT_WEIGHT_T])
def test_quantize_weight_bit_exact(kind):
    W = bf16_test_matrix((3, 256, 384), 2)
    q, s = B.quantize_fp8(W.to(DEV), kind)
    q, s = q.cpu(), s.cpu().numpy().astype(np.float64)
    for e in range(3):
        ref = O.quant_weight_128x128(W[e].float().numpy())
        if kind == B.QUANT_WEIGHT_T:
            ref = ref.T
        got = _decode(q[e], np.kron(s[e], np.ones((128, 128))))
        assert np.array_equal(got, ref), e


@pytest.mark.parametrize("gather", [True, False])
def test_quantize_tokens_bit_exact(gather):
    """Runs of 128 expert-sorted rows per column, counted from each expert's
    first row, with experts that are empty, shorter than a run, or ragged."""
    T, E, k, C = 700, 8, 2, 256
    g = np.random.default_rng(3)
    pool = np.array([0, 1, 2, 4])                           # experts 3 and 5 stay empty
    ids = np.stack([g.permutation(pool)[:k] for _ in range(T)])
    ids[:40] = [7, 6]                                       # experts 6, 7: 40 rows each
    ids = torch.from_numpy(ids.astype(np.int32))
    w = torch.from_numpy(g.uniform(0.1, 1.0, (T, k)).astype(np.float32))
    r = B.route_ids(ids.to(DEV), w.to(DEV), E)
    R = T * k
    src = bf16_test_matrix((T if gather else R, C), 4)
    q, s = B.quantize_tokens_fp8(src.to(DEV), r, T, k, gather)
    q, s = q.cpu(), s.cpu().numpy().astype(np.float64)
    rt = O.route(None, k, E, ids=ids.numpy(), w=w.double().numpy())
    counts, off = rt["counts"], rt["offsets"]
    assert counts[3] == 0 and counts[5] == 0 and counts[6] == 40
    rows = src.float().numpy()[rt["src_of"] // k] if gather else src.float().numpy()
    blk = 0
    for e in range(E):
        n = counts[e]
        nb = -(-n // 128)
        if n:
            ref = O.quant_tokens_128(rows[off[e]:off[e + 1]])          # [n, C]
            cols = slice(128 * blk, 128 * (blk + nb))
            got = _decode(q[:, cols], np.repeat(s[:, blk:blk + nb], 128, axis=1))   # [C, 128 nb]
            assert np.array_equal(got[:, :n], ref.T), e
            assert np.all(q[:, cols][:, n:].numpy() == 0), e
        blk += nb


def _wide_token_case(gather, seed):
    """65,536 expert-sorted rows over 8 experts and 1024 columns: the token
    quantisers then walk several 64-column chunks per work-group.  Returns
    the routing, the source matrix, the oracle's routing and a sample of 48
    columns, three in every chunk."""
    T, E, k, C = 16384, 8, 4, 1024
    g = np.random.default_rng(seed)
    ids = torch.from_numpy(np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32))
    w = torch.from_numpy(g.uniform(0.1, 1.0, (T, k)).astype(np.float32))
    r = B.route_ids(ids.to(DEV), w.to(DEV), E)
    src = bf16_test_matrix((T if gather else T * k, C), seed + 1)
    rt = O.route(None, k, E, ids=ids.numpy(), w=w.double().numpy())
    cols = [64 * j + c for j in range(C // 64) for c in (0, 37, 63)]
    return r, src, rt, cols, (T, E, k)


@pytest.mark.parametrize("gather", [True, False])
def test_quantize_tokens_bit_exact_many_column_chunks(gather):
    """Every 128-row run of a sample of columns spread over all chunks, at a
    size where each work-group encodes several column chunks in turn."""
    r, src, rt, cols, (T, E, k) = _wide_token_case(gather, 11)
    q, s = B.quantize_tokens_fp8(src.to(DEV), r, T, k, gather)
    q, s = q.cpu()[cols], s.cpu().numpy().astype(np.float64)[cols]
    rows = src.float().numpy()[rt["src_of"] // k] if gather else src.float().numpy()
    rows = rows[:, cols]
    counts, off = rt["counts"], rt["offsets"]
    blk = 0
    for e in range(E):
        n = counts[e]
        nb = -(-n // 128)
        ref = O.quant_tokens_128(rows[off[e]:off[e + 1]])
        got = _decode(q[:, 128 * blk:128 * (blk + nb)], np.repeat(s[:, blk:blk + nb], 128, axis=1))
        assert np.array_equal(got[:, :n], ref.T), e
        assert np.all(q[:, 128 * blk + n:128 * (blk + nb)].numpy() == 0), e
        blk += nb


SMALL = {
    # several tiles, ragged rows, a 128-wide feature tail (d = I = 384)
    "fp8_tiles": BASE.scaled(T=777, d=384, E=16, k=4, I=384),
    "fp8_wide": BASE.scaled(T=600, d=512, E=8, k=2, I=256),
    "fp8_one_token": BASE.scaled(T=1, d=128, E=8, k=2, I=128),
    "fp8_single_expert": BASE.scaled(T=300, d=256, E=1, k=1, I=128),
    # the skewed router (Zipf bias, empty experts) at a small hidden size
    "fp8_skew_small": S.WORKLOADS["fp8_skew"].scaled(T=1024, d=256, I=256),
    # the largest hidden and intermediate sizes the boundary accepts
    "fp8_max_d": BASE.scaled(T=40, d=16384, E=4, k=2, I=128),
    "fp8_max_i": BASE.scaled(T=40, d=128, E=3, k=2, I=16384),
    # few experts with many rows: every row GEMM takes its tiles
    # row-tile-major (token operands larger than the weights)
    "fp8_ep_share": BASE.scaled(T=3000, d=512, E=2, k=1, I=512),
}


# rows per expert: a whole 128-row run, one row past it, a single row, none,
# one short of two runs, two runs, one short of a run, three runs
RUN_COUNTS = [128, 129, 1, 0, 255, 256, 127, 384]


@pytest.mark.parametrize("precision", ["fp8_block", "mxfp8"])
def test_fp8_layer_run_boundaries(precision):
    """Expert segments that end exactly at, one past and one short of a
    128-row run boundary, hold one row, or none.  The token-run encodings
    (of x, dout and Aw, and of dH, which the SwiGLU backward writes itself)
    and the weight gradients over them meet the oracle at the layer
    tolerance, and the empty expert's gradients are zero."""
    counts = np.array(RUN_COUNTS)
    E, k = len(counts), 2
    T = int(counts.sum()) // k
    slots = np.repeat(np.arange(E, dtype=np.int32), counts)   # expert order
    ids = np.ascontiguousarray(np.stack([slots[:T], slots[T:]], axis=1))
    assert np.all(ids[:, 0] != ids[:, 1])                     # no expert holds T rows
    w = np.random.default_rng(8).uniform(0.1, 1.0, (T, k)).astype(np.float32)
    wl = BASE.scaled(T=T, d=256, E=E, k=k, I=256, precision=precision)
    print(f"case {precision}: {wl} counts {RUN_COUNTS}", flush=True)
    inp = S.make_inputs(wl, seed=9)
    ids_t, w_t = torch.from_numpy(ids), torch.from_numpy(w)
    gpu = run_gpu(wl, inp, ids=ids_t, w=w_t)
    ref = run_oracle(wl, inp, ids=ids_t, w=w_t)
    assert np.array_equal(ref["rt"]["counts"], counts)
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL["fp8"])
    assert np.all(gpu["dW_gate_up"][3] == 0) and np.all(gpu["dW_down"][3] == 0)
    print(precision, errs)


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_layer_parity_small(name):
    wl = SMALL[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=1)
    gpu = run_gpu(wl, inp)
    ref = run_oracle(wl, inp)
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL["fp8"])
    print(name, errs)


def test_fp8_layer_parity_full_size_sampled():
    """Skewed-routing fp8 layer at 16,384 tokens, d=4096, I=1536 in the
    benchmark's launch configuration: routing bit-exact (hot and empty
    experts), out/dx/top-k-weight/logit gradients on sampled tokens, weight
    gradients of the smallest non-empty expert, a mid-sized one and the
    hottest one (about ten times the mean load, many row tiles and token
    runs)."""
    wl = S.WORKLOADS["fp8_skew"]
    inp = S.make_inputs(wl, seed=0)
    gpu = run_gpu(wl, inp)
    lg = inp["logits"].double().numpy()
    rt = O.route(lg, wl.k, wl.E)
    check_routing(gpu, {"rt": rt})
    counts = rt["counts"]
    assert (counts == 0).sum() >= 4 and counts.max() >= 8 * counts.mean()
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    x, dout = inp["x"].double().numpy(), inp["dout"].double().numpy()
    toks = np.random.default_rng(0).choice(wl.T, 12, replace=False)
    toks[:2] = [0, wl.T - 1]
    s = O.forward_backward_tokens_fp8(x, lg, dout, Wgu, Wd, wl.k, toks)
    for n in ("out", "dx", "d_topk_w", "dlogits"):
        e = rel_err(gpu[n][toks], s[n])
        print(n, e)
        assert e <= TOL["fp8"], (n, e)
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz])]
    assert counts[order[-1]] >= 8 * counts.mean()
    for e in (order[0], order[len(order) // 2], order[-1]):
        dgu, dd = O.expert_weight_grads_fp8(x, dout, rt, Wgu, Wd, e)
        for n, got, ref in (("dW_gate_up", gpu["dW_gate_up"][e], dgu), ("dW_down", gpu["dW_down"][e], dd)):
            err = rel_err(got, ref)
            print(n, e, counts[e], err)
            assert err <= TOL["fp8"], (n, e, err)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(gpu["dW_gate_up"][e] == 0) and np.all(gpu["dW_down"][e] == 0)


# ------------------------------------------------------------ fp8_bwd option
# bf16 forward (H, Aw stored in bf16), blockwise fp8 backward on them; the
# backward encodes the weights itself.
FP8_BWD = {
    "fp8bwd_tiles": SMALL["fp8_tiles"].scaled(precision="fp8_bwd"),
    "fp8bwd_one_token": SMALL["fp8_one_token"].scaled(precision="fp8_bwd"),
    "fp8bwd_skew_small": S.WORKLOADS["fp8_bwd_skew"].scaled(T=1024, d=256, I=256),
    "fp8bwd_max_d": SMALL["fp8_max_d"].scaled(precision="fp8_bwd"),
    "fp8bwd_max_i": SMALL["fp8_max_i"].scaled(precision="fp8_bwd"),
}


@pytest.mark.parametrize("name", list(FP8_BWD))
def test_fp8_bwd_layer_parity_small(name):
    wl = FP8_BWD[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=2)
    gpu = run_gpu(wl, inp)
    ref = run_oracle(wl, inp)
    check_routing(gpu, ref)
    assert rel_err(gpu["out"], ref["out"]) <= TOL["bf16"]
    errs = check_floats(gpu, ref, TOL["fp8"])
    print(name, errs)


def test_fp8_bwd_layer_parity_full_size_sampled():
    """fp8_bwd on the skewed layer at 16,384 tokens, d=4096, I=1536: sampled
    tokens and two experts' weight gradients, as for fp8."""
    wl = S.WORKLOADS["fp8_bwd_skew"]
    inp = S.make_inputs(wl, seed=0)
    gpu = run_gpu(wl, inp)
    lg = inp["logits"].double().numpy()
    rt = O.route(lg, wl.k, wl.E)
    check_routing(gpu, {"rt": rt})
    counts = rt["counts"]
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    x, dout = inp["x"].double().numpy(), inp["dout"].double().numpy()
    toks = np.random.default_rng(1).choice(wl.T, 12, replace=False)
    toks[:2] = [0, wl.T - 1]
    s = O.forward_backward_tokens_fp8(x, lg, dout, Wgu, Wd, wl.k, toks, fwd_recipe=O.NO_QUANT)
    for n in ("out", "dx", "d_topk_w", "dlogits"):
        e = rel_err(gpu[n][toks], s[n])
        print(n, e)
        assert e <= TOL["bf16" if n == "out" else "fp8"], (n, e)
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz])]
    for e in (order[0], order[-1]):
        dgu, dd = O.expert_weight_grads_fp8(x, dout, rt, Wgu, Wd, e, fwd_recipe=O.NO_QUANT)
        for n, got, ref in (("dW_gate_up", gpu["dW_gate_up"][e], dgu), ("dW_down", gpu["dW_down"][e], dd)):
            err = rel_err(got, ref)
            print(n, e, counts[e], err)
            assert err <= TOL["fp8"], (n, e, err)
