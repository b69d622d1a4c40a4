"""MXFP8 path (OCP e4m3 in blocks of 32 with E8M0 power-of-two scales)
against the oracle.

Quantisation is byte work and must match bit for bit: every e4m3 code and
every scale byte.  Layer outputs and gradients match the oracle's emulation
of the same quantisation within max|err|/max|ref| <= 6e-2.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from combine_top_route_amd import binding as B
from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O

from gpu_util import TOL, bf16_test_matrix, check_floats, check_routing, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
MX = dict(dtype="bf16", logits_dtype="bf16", precision="mxfp8")
BASE = S.WORKLOADS["tiny"].scaled(**MX)


def _codes(values):
    """e4m3 codes of values that are already e4m3 numbers (exact cast)."""
    return torch.from_numpy(np.ascontiguousarray(values)).to(torch.float8_e4m3fn).view(torch.uint8)


def _check_encoding(q, s, X):
    """q, s: the library's codes and scale bytes of X encoded in 1 x 32
    blocks along its last axis."""
    ref_q, ref_x = O.mx_quant_last(X)
    assert torch.equal(q.cpu(), _codes(ref_q)), "codes"
    assert np.array_equal(s.cpu().numpy().astype(np.int64), ref_x + 127), "scale bytes"


def test_mx_quantize_rows_bit_exact():
    x = bf16_test_matrix((300, 512), 1)
    q, s = B.quantize_mxfp8(x.to(DEV), B.QUANT_ROWS)
    _check_encoding(q, s, x.float().numpy())


@pytest.mark.parametrize("kind", [B.QUANT_WEIGHT, B.QUANT_WEIGHT_T])
def test_mx_quantize_weight_bit_exact(kind):
    """Forward encoding: blocks along each row; data-gradient encoding:
    blocks down each column, written transposed."""
    W = bf16_test_matrix((3, 256, 384), 2)
    q, s = B.quantize_mxfp8(W.to(DEV), kind)
    for e in range(3):
        M = W[e].float().numpy()
        _check_encoding(q[e], s[e], M if kind == B.QUANT_WEIGHT else M.T.copy())


@pytest.mark.parametrize("gather", [True, False])
def test_mx_quantize_tokens_bit_exact(gather):
    """32-row blocks inside 128-row runs of each expert's segment, counted
    from the expert's first row; experts empty, shorter than a block, or
    ragged."""
    T, E, k, C = 700, 8, 2, 256
    g = np.random.default_rng(3)
    pool = np.array([0, 1, 2, 4])                           # experts 3 and 5 stay empty
    ids = np.stack([g.permutation(pool)[:k] for _ in range(T)])
    ids[:40] = [7, 6]                                       # experts 6, 7: 40 rows each
    ids[40:45] = [5, 6]                                     # expert 5: 5 rows
    ids = torch.from_numpy(ids.astype(np.int32))
    w = torch.from_numpy(g.uniform(0.1, 1.0, (T, k)).astype(np.float32))
    r = B.route_ids(ids.to(DEV), w.to(DEV), E)
    R = T * k
    src = bf16_test_matrix((T if gather else R, C), 4)
    q, s = B.quantize_tokens_mxfp8(src.to(DEV), r, T, k, gather)
    q, s = q.cpu(), s.cpu()
    rt = O.route(None, k, E, ids=ids.numpy(), w=w.double().numpy())
    counts, off = rt["counts"], rt["offsets"]
    assert counts[3] == 0 and counts[5] == 5 and counts[6] == 45
    rows = src.float().numpy()[rt["src_of"] // k] if gather else src.float().numpy()
    blk = 0
    for e in range(E):
        n = counts[e]
        nb = -(-n // 128)
        if n:
            pad = np.zeros((128 * nb, C), np.float32)
            pad[:n] = rows[off[e]:off[e + 1]]
            _check_encoding(q[:, 128 * blk:128 * (blk + nb)], s[:, 4 * blk:4 * (blk + nb)], pad.T.copy())
            # the same values as the oracle's token blocks of the segment alone
            ref_q, ref_x = O.mx_quant_last(pad.T.copy())
            deq = np.ldexp(ref_q, np.repeat(ref_x, 32, axis=1))[:, :n]
            assert np.array_equal(deq, O.mx_tokens(rows[off[e]:off[e + 1]]).T)
        blk += nb


@pytest.mark.parametrize("gather", [True, False])
def test_mx_quantize_tokens_bit_exact_many_column_chunks(gather):
    """Every 32-row block of a sample of columns spread over all 64-column
    chunks, at a size where each work-group encodes several chunks in turn
    (65,536 expert-sorted rows, 1024 columns)."""
    T, E, k, C = 16384, 8, 4, 1024
    g = np.random.default_rng(13)
    ids = torch.from_numpy(np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32))
    w = torch.from_numpy(g.uniform(0.1, 1.0, (T, k)).astype(np.float32))
    r = B.route_ids(ids.to(DEV), w.to(DEV), E)
    src = bf16_test_matrix((T if gather else T * k, C), 14)
    q, s = B.quantize_tokens_mxfp8(src.to(DEV), r, T, k, gather)
    cols = [64 * j + c for j in range(C // 64) for c in (0, 37, 63)]
    q, s = q.cpu()[cols], s.cpu()[cols]
    rt = O.route(None, k, E, ids=ids.numpy(), w=w.double().numpy())
    rows = src.float().numpy()[rt["src_of"] // k] if gather else src.float().numpy()
    rows = rows[:, cols]
    counts, off = rt["counts"], rt["offsets"]
    blk = 0
    for e in range(E):
        n = counts[e]
        nb = -(-n // 128)
        pad = np.zeros((128 * nb, len(cols)), np.float32)
        pad[:n] = rows[off[e]:off[e + 1]]
        _check_encoding(q[:, 128 * blk:128 * (blk + nb)], s[:, 4 * blk:4 * (blk + nb)], pad.T.copy())
        blk += nb


SMALL = {
    # several tiles, ragged rows, a 128-wide feature tail (d = I = 384)
    "mx_tiles": BASE.scaled(T=777, d=384, E=16, k=4, I=384),
    "mx_wide": BASE.scaled(T=600, d=512, E=8, k=2, I=256),
    "mx_one_token": BASE.scaled(T=1, d=128, E=8, k=2, I=128),
    "mx_single_expert": BASE.scaled(T=300, d=256, E=1, k=1, I=128),
    # the skewed router (Zipf bias, empty experts) at a small hidden size
    "mx_skew_small": S.WORKLOADS["mxfp8_skew"].scaled(T=1024, d=256, I=256),
    # the largest hidden and intermediate sizes the boundary accepts
    "mx_max_d": BASE.scaled(T=40, d=16384, E=4, k=2, I=128),
    "mx_max_i": BASE.scaled(T=40, d=128, E=3, k=2, I=16384),
    # few experts with many rows: every row GEMM takes its tiles
    # row-tile-major (token operands larger than the weights)
    "mx_ep_share": BASE.scaled(T=3000, d=512, E=2, k=1, I=512),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_mx_layer_parity_small(name):
    wl = SMALL[name]
    print(f"case {name}: {wl}", flush=True)
    inp = S.make_inputs(wl, seed=1)
    gpu = run_gpu(wl, inp)
    ref = run_oracle(wl, inp)
    check_routing(gpu, ref)
    errs = check_floats(gpu, ref, TOL["fp8"])
    print(name, errs)


def test_mx_layer_parity_full_size_sampled():
    """Skewed-routing MXFP8 layer at 16,384 tokens, d=4096, I=1536 in the
    benchmark's launch configuration: routing bit-exact, out/dx/top-k-weight/
    logit gradients on sampled tokens, weight gradients of the smallest
    non-empty expert, a mid-sized one and the hottest one (about ten times
    the mean load), zeros for empty experts.  The oracle encodes each touched
    expert's weights four ways (a few seconds per expert), so the sampled
    tokens are the first and last ones plus tokens routed only to the eight
    busiest experts and 24 experts drawn at random from the non-empty ones:
    about twenty experts whose loads span the whole range, hot to cold."""
    wl = S.WORKLOADS["mxfp8_skew"]
    inp = S.make_inputs(wl, seed=0)
    gpu = run_gpu(wl, inp)
    lg = inp["logits"].double().numpy()
    rt = O.route(lg, wl.k, wl.E)
    check_routing(gpu, {"rt": rt})
    counts = rt["counts"]
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    x, dout = inp["x"].double().numpy(), inp["dout"].double().numpy()
    ids = rt["ids"]
    g = np.random.default_rng(0)
    busiest = np.argsort(-counts, kind="stable")[:8]
    drawn = g.choice(np.nonzero(counts)[0], 24, replace=False)
    allowed = set(busiest.tolist()) | set(drawn.tolist()) | set(ids[0].tolist()) | set(ids[-1].tolist())
    cand = [t for t in range(1, wl.T - 1) if set(ids[t].tolist()) <= allowed]
    assert len(cand) >= 10, len(cand)
    toks = np.concatenate([[0, wl.T - 1], g.choice(cand, 10, replace=False)])
    used = np.unique(ids[toks])
    rank = np.argsort(np.argsort(-counts, kind="stable"), kind="stable")
    print("experts sampled", used.size, "load ranks", sorted(rank[used].tolist()))
    assert rank[used].max() >= 64          # the sample reaches the cold half of the experts
    with ThreadPoolExecutor(max_workers=8) as ex:   # the encodings, expert by expert, in parallel
        enc = dict(zip(used.tolist(), ex.map(
            lambda e: O.encode_expert_weights(Wgu, Wd, e, recipe=O.MXFP8), used.tolist())))
    s = O.forward_backward_tokens_fp8(x, lg, dout, Wgu, Wd, wl.k, toks, recipe=O.MXFP8, encoded=enc)
    for n in ("out", "dx", "d_topk_w", "dlogits"):
        e = rel_err(gpu[n][toks], s[n])
        print(n, e)
        assert e <= TOL["fp8"], (n, e)
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz])]
    assert counts[order[-1]] >= 8 * counts.mean()
    for e in (order[0], order[len(order) // 2], order[-1]):
        dgu, dd = O.expert_weight_grads_fp8(x, dout, rt, Wgu, Wd, e, recipe=O.MXFP8)
        for n, got, ref in (("dW_gate_up", gpu["dW_gate_up"][e], dgu), ("dW_down", gpu["dW_down"][e], dd)):
            err = rel_err(got, ref)
            print(n, e, counts[e], err)
            assert err <= TOL["fp8"], (n, e, err)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(gpu["dW_gate_up"][e] == 0) and np.all(gpu["dW_down"][e] == 0)
