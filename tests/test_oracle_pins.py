"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a library routine, a closed form, a
brute-force evaluation, finite differences or an invariant, chosen so that a
plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, gate and up swapped) fails at least one of them.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O


def _np(t):
    return t.double().numpy()


def _tiny(seed=0, **kw):
    wl = S.WORKLOADS["tiny"].scaled(**kw)
    inp = S.make_inputs(wl, seed=seed)
    return wl, {k: _np(v) for k, v in inp.items()}


# ---------------------------------------------------------------- routing

def test_topk_matches_stable_argsort_on_bf16_ties():
    # bf16 logits tie often; numpy's stable argsort of -l is the library
    # statement of "largest first, ties to the lower index".
    wl = S.WORKLOADS["q30b"]
    lg = _np(S.make_logits(wl, seed=3, T=2048))
    ids = O.topk_select(lg, 8)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref)
    # the data really contains ties at the selection boundary
    srt = -np.sort(-lg, axis=1)
    assert np.mean(srt[:, 7] == srt[:, 8]) > 0.01


def test_topk_bruteforce_python_loops():
    rng = np.random.default_rng(1)
    lg = np.round(rng.standard_normal((40, 9)), 1)        # many exact ties
    k = 4
    ids = O.topk_select(lg, k)
    for t in range(lg.shape[0]):
        remaining = list(range(lg.shape[1]))
        for j in range(k):
            best = remaining[0]
            for e in remaining:
                if lg[t, e] > lg[t, best]:
                    best = e
            assert ids[t, j] == best
            remaining.remove(best)


def test_topk_tie_rules_explicit():
    lg = np.array([[1.0, 2.0, 2.0, 0.5],
                   [0.0, -0.0, 0.0, -1.0],
                   [-np.inf, -np.inf, 3.0, -np.inf]])
    ids = O.topk_select(lg, 3)
    assert ids[0].tolist() == [1, 2, 0]
    assert ids[1].tolist() == [0, 1, 2]          # -0.0 ties with +0.0
    assert ids[2].tolist() == [2, 0, 1]          # all -inf: lower index first


def test_weights_closed_form_and_full_softmax():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((64, 16)) * 3
    ids = O.topk_select(lg, 5)
    w = O.topk_weights(lg, ids)
    full = np.exp(lg - lg.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 1e-15)    # slot order = weight order
    # k = 2 closed form: w0 = 1 / (1 + exp(l1 - l0))
    ids2 = O.topk_select(lg, 2)
    w2 = O.topk_weights(lg, ids2)
    l0 = np.take_along_axis(lg, ids2[:, :1], 1)[:, 0]
    l1 = np.take_along_axis(lg, ids2[:, 1:], 1)[:, 0]
    np.testing.assert_allclose(w2[:, 0], 1 / (1 + np.exp(l1 - l0)), rtol=1e-13)


def test_counts_offsets_permutation_invariants_and_bruteforce():
    wl, inp = _tiny()
    rt = O.route(inp["logits"], wl.k, wl.E)
    T, k, E, R = wl.T, wl.k, wl.E, wl.R
    c, off, src, row = rt["counts"], rt["offsets"], rt["src_of"], rt["row_of"]
    assert c.sum() == R and off[0] == 0 and off[E] == R
    assert np.array_equal(np.sort(src), np.arange(R))
    assert np.array_equal(row[src], np.arange(R))
    flat = rt["ids"].ravel()
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)          # token order inside an expert
    # O(T*k*E) brute force of the dispatch order
    expect = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if rt["ids"][t, j] == e:
                    expect.append(t * k + j)
    assert np.array_equal(src, np.array(expect))
    c2, off2 = O.expert_counts(rt["ids"], E)
    assert np.array_equal(c2, c) and np.array_equal(off2, off)


# ---------------------------------------------------------------- forward

def _dense_bruteforce(x, lg, Wgu, Wd, k):
    """Every token through every expert, masked by its top-k gate."""
    T, E = lg.shape
    I = Wgu.shape[1] // 2
    out = np.zeros((T, Wd.shape[1]))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        z = np.array([math.exp(lg[t, e] - lg[t, order[0]]) for e in order])
        gate = dict(zip(order, z / z.sum()))
        for e in range(E):
            g = Wgu[e, :I] @ x[t]
            u = Wgu[e, I:] @ x[t]
            a = g / (1 + np.exp(-g)) * u
            y = Wd[e] @ a
            out[t] += gate.get(e, 0.0) * y
    return out


def test_forward_dense_bruteforce():
    wl, inp = _tiny(seed=4, T=48)
    rt = O.route(inp["logits"], wl.k, wl.E)
    fw = O.forward(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    ref = _dense_bruteforce(inp["x"], inp["logits"], inp["w_gate_up"], inp["w_down"], wl.k)
    np.testing.assert_allclose(fw["out"], ref, rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_swiglu_mlp_torch():
    # E = 1, k = 1: the layer is a dense SwiGLU MLP (torch CPU ops)
    rng = np.random.default_rng(5)
    T, d, I = 33, 24, 40
    x = rng.standard_normal((T, d))
    Wgu = rng.standard_normal((1, 2 * I, d)) / math.sqrt(d)
    Wd = rng.standard_normal((1, d, I)) / math.sqrt(I)
    lg = rng.standard_normal((T, 1))
    rt = O.route(lg, 1, 1)
    out = O.forward(x, rt, Wgu, Wd)["out"]
    xt = torch.from_numpy(x)
    gate = torch.nn.functional.linear(xt, torch.from_numpy(Wgu[0, :I]))
    up = torch.nn.functional.linear(xt, torch.from_numpy(Wgu[0, I:]))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up,
                                     torch.from_numpy(Wd[0]))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_hand_worked_example():
    """T=2, d=2, E=3, k=2, I=1 with values worked out by hand.

    token 0: logits (1, 0, 1): experts 0 and 2 tie, order (0, 2), w = (1/2, 1/2)
    token 1: logits (0, ln 3, -1): order (1, 0), w = (3/4, 1/4)
    expert e: gate row a_e, up row c_e of W_gate_up; W_down column p_e.
    """
    x = np.array([[1.0, 0.0], [0.0, 2.0]])
    lg = np.array([[1.0, 0.0, 1.0], [0.0, math.log(3.0), -1.0]])
    Wgu = np.array([[[2.0, 1.0], [3.0, -1.0]],     # e0: gate (2,1), up (3,-1)
                    [[0.5, 0.0], [1.0, 1.0]],      # e1
                    [[-1.0, 4.0], [0.0, 2.0]]])    # e2
    Wd = np.array([[[1.0], [2.0]], [[-1.0], [0.5]], [[3.0], [1.0]]])
    rt = O.route(lg, 2, 3)
    assert rt["ids"].tolist() == [[0, 2], [1, 0]]
    np.testing.assert_allclose(rt["w"], [[0.5, 0.5], [0.75, 0.25]], rtol=1e-15)
    assert rt["counts"].tolist() == [2, 1, 1]
    assert rt["src_of"].tolist() == [0, 3, 2, 1]   # e0: (t0,j0),(t1,j1); e1: (t1,j0); e2: (t0,j1)

    def silu(z):
        return z / (1 + math.exp(-z))
    # token 0: e0 -> g = 2, u = 3, a = 3 silu(2); e2 -> g = -1, u = 0, a = 0
    y00 = 3 * silu(2.0) * np.array([1.0, 2.0])
    out0 = 0.5 * y00
    # token 1 (x = (0, 2)): e1 -> g = 0 -> a = 0; e0 -> g = 2, u = -2, a = -2 silu(2)
    y10 = -2 * silu(2.0) * np.array([1.0, 2.0])
    out1 = 0.25 * y10
    fw = O.forward(x, rt, Wgu, Wd)
    np.testing.assert_allclose(fw["out"], np.stack([out0, out1]), rtol=1e-14)


def test_identity_experts_return_input():
    wl, inp = _tiny(seed=6)
    x = inp["x"]
    # k = 1, w = 1: exactly x, bit for bit
    ids, _ = S.random_topk(wl.T, wl.E, 1, seed=6)
    rt = O.route(None, 1, wl.E, ids=ids.numpy(), w=np.ones((wl.T, 1)))
    out = O.forward(x, rt, None, None, expert_fn=lambda e, xp: xp)["out"]
    assert np.array_equal(out, x)
    # general k with renormalised weights: x up to rounding
    rt = O.route(inp["logits"], wl.k, wl.E)
    out = O.forward(x, rt, None, None, expert_fn=lambda e, xp: xp)["out"]
    np.testing.assert_allclose(out, x, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- backward

def _loss(x, rt, Wgu, Wd, dout):
    return float(np.sum(dout * O.forward(x, rt, Wgu, Wd)["out"]))


def test_backward_finite_differences():
    wl, inp = _tiny(seed=7, T=32)
    x, lg, Wgu, Wd, dout = (inp[n] for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    rt = O.route(lg, wl.k, wl.E)
    fw = O.forward(x, rt, Wgu, Wd)
    g = O.backward(dout, rt, Wgu, Wd, fw, logits=lg)
    rng = np.random.default_rng(8)
    h = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("Wgu", Wgu, g["dW_gate_up"]),
                            ("Wd", Wd, g["dW_down"])):
        for _ in range(3):
            v = rng.standard_normal(arr.shape)
            args = dict(x=x, Wgu=Wgu, Wd=Wd)
            args[name] = arr + h * v
            lp = _loss(args["x"], rt, args["Wgu"], args["Wd"], dout)
            args[name] = arr - h * v
            lm = _loss(args["x"], rt, args["Wgu"], args["Wd"], dout)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grad * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # every top-k weight, in ids-in mode
    for t in range(0, wl.T, 5):
        for j in range(wl.k):
            wp = rt["w"].copy(); wp[t, j] += h
            wm = rt["w"].copy(); wm[t, j] -= h
            rp = O.route(None, wl.k, wl.E, ids=rt["ids"], w=wp)
            rm = O.route(None, wl.k, wl.E, ids=rt["ids"], w=wm)
            fd = (_loss(x, rp, Wgu, Wd, dout) - _loss(x, rm, Wgu, Wd, dout)) / (2 * h)
            assert abs(fd - g["d_topk_w"][t, j]) <= 1e-6 * max(1.0, abs(fd))
    # logits: directions that leave every token's selection unchanged
    for _ in range(3):
        v = rng.standard_normal(lg.shape)
        rp = O.route(lg + h * v, wl.k, wl.E)
        rm = O.route(lg - h * v, wl.k, wl.E)
        assert np.array_equal(rp["ids"], rt["ids"]) and np.array_equal(rm["ids"], rt["ids"])
        fd = (_loss(x, rp, Wgu, Wd, dout) - _loss(x, rm, Wgu, Wd, dout)) / (2 * h)
        an = float(np.sum(g["dlogits"] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_empty_expert_gets_zero_weight_grad():
    wl, inp = _tiny(seed=9, T=16)
    ids, w = S.random_topk(wl.T, wl.E - 1, wl.k, seed=9)
    ids = ids.numpy()
    ids = ids + (ids >= 3)                   # skip expert 3: it receives nothing
    rt = O.route(None, wl.k, wl.E, ids=ids, w=w.numpy())
    fw = O.forward(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    g = O.backward(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], fw)
    assert rt["counts"][3] == 0
    assert np.all(g["dW_gate_up"][3] == 0) and np.all(g["dW_down"][3] == 0)
    assert np.any(g["dW_gate_up"][2] != 0)


def test_sampled_evaluation_matches_full():
    wl, inp = _tiny(seed=10)
    x, lg, Wgu, Wd, dout = (inp[n] for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    rt = O.route(lg, wl.k, wl.E)
    fw = O.forward(x, rt, Wgu, Wd)
    g = O.backward(dout, rt, Wgu, Wd, fw, logits=lg)
    toks = np.array([0, 5, 77, 127])
    s = O.forward_backward_tokens(x, lg, dout, Wgu, Wd, wl.k, toks)
    for n in ("out",):
        np.testing.assert_allclose(s[n], fw[n][toks], rtol=1e-12, atol=1e-12)
    for n in ("dx", "d_topk_w", "dlogits"):
        np.testing.assert_allclose(s[n], g[n][toks], rtol=1e-12, atol=1e-12)
    for e in (0, 3):
        dgu, dd = O.expert_weight_grads(x, dout, rt, Wgu, Wd, e)
        np.testing.assert_allclose(dgu, g["dW_gate_up"][e], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dd, g["dW_down"][e], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """A dropped term in the SwiGLU backward, or gate/up swapped, must break
    the pins above (finite differences / torch dense MLP)."""
    wl, inp = _tiny(seed=11, T=16)
    x, lg, Wgu, Wd, dout = (inp[n] for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    rt = O.route(lg, wl.k, wl.E)

    def fd_gap():
        fw = O.forward(x, rt, Wgu, Wd)
        g = O.backward(dout, rt, Wgu, Wd, fw)
        v = np.random.default_rng(0).standard_normal(x.shape)
        h = 1e-6
        fd = (_loss(x + h * v, rt, Wgu, Wd, dout) - _loss(x - h * v, rt, Wgu, Wd, dout)) / (2 * h)
        return abs(fd - float(np.sum(g["dx"] * v)))

    assert fd_gap() < 1e-6
    real = O.swiglu_backward

    def dropped(H, dA, I, limit=0.0):
        g, u = H[:, :I], H[:, I:]
        s = O.sigmoid(g)
        return np.concatenate([dA * u * s, dA * g * s], axis=1)   # missing (1 + g(1-s))
    monkeypatch.setattr(O, "swiglu_backward", dropped)
    assert fd_gap() > 1e-3
    monkeypatch.setattr(O, "swiglu_backward", real)

    def swapped(H, I, limit=0.0):
        return O.silu(H[:, I:]) * H[:, :I]
    monkeypatch.setattr(O, "swiglu", swapped)
    rng = np.random.default_rng(5)
    xx = rng.standard_normal((4, 6))
    W1 = rng.standard_normal((1, 8, 6))
    W2 = rng.standard_normal((1, 6, 4))
    out = O.forward(xx, O.route(np.zeros((4, 1)), 1, 1), W1, W2)["out"]
    xt = torch.from_numpy(xx)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(xt @ torch.from_numpy(W1[0, :4]).T) * (xt @ torch.from_numpy(W1[0, 4:]).T),
        torch.from_numpy(W2[0]))
    assert not np.allclose(out, ref.numpy(), rtol=1e-6)


# ---------------------------------------------------------------- fp8

def test_e4m3_round_matches_torch_cast_on_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    ours = O.e4m3_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_bounds():
    assert O.e4m3_round(np.array([500.0, -1e6, 464.0]))[:].tolist() == [448.0, -448.0, 448.0]
    rng = np.random.default_rng(12)
    v = rng.standard_normal(100000) * 50
    q = O.e4m3_round(v)
    nrm = np.abs(v) >= 2.0 ** -6
    assert np.all(np.abs(q[nrm] - v[nrm]) <= np.abs(v[nrm]) * 2.0 ** -4 + 1e-300)
    assert np.all(np.abs(q[~nrm] - v[~nrm]) <= 2.0 ** -10)


def test_block_quantisers_exact_on_representable_blocks():
    rng = np.random.default_rng(13)
    # every value an e4m3 number times 2^-3, with +-448 * 2^-3 in every block
    grid = O.e4m3_round(rng.standard_normal((4, 256)) * 60) * 2.0 ** -3
    grid[:, 0] = 448 * 2.0 ** -3
    grid[:, 128] = -448 * 2.0 ** -3
    assert np.array_equal(O.quant_rows_1x128(grid), grid)
    assert np.array_equal(O.quant_tokens_128(grid.T.copy()), grid.T)
    W = np.tile(grid, (64, 1))[:256]
    assert np.array_equal(O.quant_weight_128x128(W), W)


def test_block_quantiser_scale_is_per_block():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((3, 384))
    q = O.quant_rows_1x128(X)
    X2 = X.copy()
    X2[1, 130] = 1000.0                         # only block (1, 1) changes
    q2 = O.quant_rows_1x128(X2)
    same = np.ones_like(X, bool)
    same[1, 128:256] = False
    assert np.array_equal(q[same], q2[same])
    assert not np.array_equal(q[1, 128:256], q2[1, 128:256])
    # the largest element of each block survives exactly
    for r in range(3):
        for c0 in range(0, 384, 128):
            i = np.argmax(np.abs(X[r, c0:c0 + 128]))
            assert abs(q[r, c0 + i] - np.float32(X[r, c0 + i])) <= 1e-6 * abs(X[r, c0 + i])


def test_fp8_layer_close_to_unquantised_layer():
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=256, T=64, dtype="bf16")
    inp = {k: _np(v) for k, v in S.make_inputs(wl, seed=15).items()}
    rt = O.route(inp["logits"], wl.k, wl.E)
    fw = O.forward(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    bw = O.backward(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], fw)
    f8 = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    b8 = O.backward_fp8(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], f8)
    for ref, got in ((fw["out"], f8["out"]), (bw["dx"], b8["dx"]),
                     (bw["dW_gate_up"], b8["dW_gate_up"]), (bw["dW_down"], b8["dW_down"]),
                     (bw["d_topk_w"], b8["d_topk_w"])):
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        assert 1e-3 < err < 0.1


def test_fp8_gate_up_exact_on_representable_operands():
    """x and W_gate_up already on the e4m3 grid of their blocks (each block's
    largest magnitude 448 * 2^-s): quantisation is the identity, so the fp8
    pre-activations equal the bf16-rounded exact product."""
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=128, T=40, E=4, k=2, dtype="bf16")
    rng = np.random.default_rng(16)
    x = O.e4m3_round(rng.standard_normal((wl.T, wl.d)) * 60) * 2.0 ** -4
    x[:, 0], x[:, 128] = 448 * 2.0 ** -4, -448 * 2.0 ** -4
    W = O.e4m3_round(rng.standard_normal((wl.E, 2 * wl.I, wl.d)) * 60) * 2.0 ** -9
    W[:, 0::128, 0::128] = 448 * 2.0 ** -9
    Wd = rng.standard_normal((wl.E, wl.d, wl.I)) * 0.05
    rt = O.route(rng.standard_normal((wl.T, wl.E)), wl.k, wl.E)
    f8 = O.forward_fp8(x, rt, W, Wd)
    H = np.concatenate([O.dispatch(x, rt)[s0:s1] @ W[e].T for e, (s0, s1) in
                        enumerate(zip(rt["offsets"][:-1], rt["offsets"][1:]))])
    assert np.array_equal(f8["H"], O.bf16_round(H))


def test_fp8_sampled_evaluators_match_full_layer():
    """The per-token and per-expert fp8 evaluators reproduce forward_fp8 /
    backward_fp8 (same arithmetic, different grouping)."""
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=128, T=96, E=6, k=2, dtype="bf16")
    inp = {k: _np(v) for k, v in S.make_inputs(wl, seed=17).items()}
    rt = O.route(inp["logits"], wl.k, wl.E)
    f8 = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    b8 = O.backward_fp8(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], f8, logits=inp["logits"])
    toks = np.array([0, 5, 50, 95])
    s = O.forward_backward_tokens_fp8(inp["x"], inp["logits"], inp["dout"], inp["w_gate_up"],
                                      inp["w_down"], wl.k, toks)
    for n, ref in (("out", f8["out"]), ("dx", b8["dx"]), ("d_topk_w", b8["d_topk_w"]),
                   ("dlogits", b8["dlogits"])):
        np.testing.assert_allclose(s[n], ref[toks], rtol=1e-12, atol=1e-12 * np.max(np.abs(ref)))
    for e in range(wl.E):
        dgu, dd = O.expert_weight_grads_fp8(inp["x"], inp["dout"], rt, inp["w_gate_up"], inp["w_down"], e)
        np.testing.assert_allclose(dgu, b8["dW_gate_up"][e], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dd, b8["dW_down"][e], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- MXFP8

def _mx_block(head):
    b = np.zeros(32)
    b[:len(head)] = head
    return b


def test_mx_hand_worked_blocks():
    """Blocks worked by hand: X is the smallest integer with amax <= 448 *
    2^X, elements are rounded to nearest e4m3 (ties to even) after dividing
    by 2^X."""
    X = np.stack([
        # amax 3 = 1.5 * 2^1 -> X = -7, so values are multiples of 2^-7 on
        # e4m3's grid: 3*128 = 384 exact; 0.1*128 = 12.8 -> 13; 0.02*128 =
        # 2.56 -> 2.5 (quantum 1/4 in [2, 4)); -2.9*128 = -371.2 -> -384
        # (quantum 32 in [256, 512))
        _mx_block([3.0, 0.1, 0.02, -2.9]),
        # amax 1.9 > 1.75 * 2^0 -> X = -7: 1.9*128 = 243.2 -> 240 (quantum
        # 16); 1.0625*128 = 136 ties between 128 (even) and 144 -> 128;
        # 1.1875*128 = 152 ties between 144 and 160 (even) -> 160; 0.75*128
        # = 96 exact
        _mx_block([1.9, 1.0625, 1.1875, 0.75]),
        # amax exactly 448 * 2^-8 -> X = -8, no rounding up
        _mx_block([1.75, -0.3]),
        np.zeros(32),                              # all zero -> X = 0
        # amax 2^-130 (an fp32 subnormal) -> X clamps at -127: 2^-3 exact,
        # 2^-135 -> 2^-8 exact (e4m3 subnormal), 3*2^-138 = 0.75*2^-9 -> 2^-9
        _mx_block([2.0 ** -130, 2.0 ** -135, 3 * 2.0 ** -138]),
    ])
    q, ex = O.mx_quant_last(X.reshape(1, -1))
    assert ex.ravel().tolist() == [-7, -7, -8, 0, -127]
    got = O.mx_rows(X)
    want = np.stack([
        _mx_block([3.0, 13 / 128, 2.5 / 128, -3.0]),
        _mx_block([240 / 128, 1.0, 1.25, 0.75]),
        # -0.3*256 = -76.8 -> -80 (quantum 8 in [64, 128))
        _mx_block([1.75, -80 / 256]),
        np.zeros(32),
        _mx_block([2.0 ** -130, 2.0 ** -135, 2.0 ** -136]),
    ])
    x32 = X.astype(np.float32).astype(np.float64)    # 0.1, 0.02, 2.9 as float32
    assert x32[0, 1] != 0.1
    assert np.array_equal(got, want)


def test_mx_scale_exponent_closed_form():
    """For every amax above the clamp, amax / 2^X lies in (224, 448]: the
    block's largest value lands in e4m3's top binade without saturating."""
    rng = np.random.default_rng(30)
    amax = (np.exp(rng.uniform(-80, 80, 100000)) * rng.choice([1, 3, 7], 100000)).astype(np.float32)
    amax = np.concatenate([amax, np.float32([1.0, 1.75, 1.7500001, 2.0, 448.0, 449.0, 2.0 ** -118])])
    X = O.mx_scale_exponent(amax)
    r = amax.astype(np.float64) / np.ldexp(1.0, X)
    assert np.all((r > 224) & (r <= 448))
    assert O.mx_scale_exponent(np.float32(0.0)) == 0
    assert O.mx_scale_exponent(np.float32(2.0 ** -125)) == -127


def test_mx_quantisers_per_block_and_exact_on_grid():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((4, 128))
    q = O.mx_rows(X)
    X2 = X.copy()
    X2[2, 70] = 1e9                                # only block (2, 64..95) changes
    q2 = O.mx_rows(X2)
    same = np.ones_like(X, bool)
    same[2, 64:96] = False
    assert np.array_equal(q[same], q2[same]) and not np.array_equal(q[2, 64:96], q2[2, 64:96])
    # any e4m3 value times a power of two whose block maximum sits in one
    # binade [1, 1.75] * 2^c is on the grid of its block, in either blocking
    v = O.e4m3_round(rng.uniform(1, 1.75, (64, 96)) * rng.choice([-1, 1], (64, 96)))
    G = v * np.ldexp(1.0, rng.integers(-20, 5, (64, 1)))  # one binade per row
    assert np.array_equal(O.mx_rows(G), G)
    assert not np.array_equal(O.mx_cols(G), G)          # columns mix binades 2^24 apart
    assert np.array_equal(O.mx_cols(G.T.copy()), G.T)


def test_mx_token_blocks_start_at_the_expert_first_row():
    """32-token blocks counted from row 0 of the segment: a large value in
    row 31 rescales rows 0..31 only; a ragged tail is its own block."""
    rng = np.random.default_rng(32)
    X = rng.standard_normal((70, 3))
    q = O.mx_tokens(X)
    X2 = X.copy()
    X2[31, 1] = 1e9                              # pushes its block into e4m3 subnormals
    q2 = O.mx_tokens(X2)
    assert np.array_equal(q2[32:], q[32:]) and np.array_equal(q2[:, [0, 2]], q[:, [0, 2]])
    assert not np.array_equal(q2[:31, 1], q[:31, 1])
    X3 = X.copy()
    X3[64, 0] = 1e9                              # rows 64..69: the short last block
    q3 = O.mx_tokens(X3)
    assert np.array_equal(q3[:64], q[:64]) and not np.array_equal(q3[65:, 0], q[65:, 0])


def _mx_axis_case(seed):
    """Tiny bf16-shaped layer whose x and dout rows sit on the e4m3 grid of
    their 1 x 32 blocks, whose W_gate_up rows and W_down columns each hold
    one binade ([1, 1.75] * 2^c with c = 0 or -20): exact in the blocking
    each GEMM should use, not in the other."""
    wl = S.WORKLOADS["tiny"].scaled(d=64, I=64, T=40, E=3, k=2, dtype="bf16")
    rng = np.random.default_rng(seed)

    def grid(shape):
        return O.e4m3_round(rng.uniform(1, 1.75, shape) * rng.choice([-1, 1], shape))
    x = grid((wl.T, wl.d))
    dout = grid((wl.T, wl.d))
    Wgu = grid((wl.E, 2 * wl.I, wl.d)) * np.ldexp(1.0, rng.choice([0, -20], (wl.E, 2 * wl.I, 1)))
    Wd = grid((wl.E, wl.d, wl.I)) * np.ldexp(1.0, rng.choice([0, -20], (wl.E, 1, wl.I)))
    rt = O.route(rng.standard_normal((wl.T, wl.E)), wl.k, wl.E)
    return wl, x, dout, Wgu, Wd, rt


def test_mx_gemm_blocking_axes():
    """Forward gate/up GEMM blocks W_gate_up along d (its rows: exact here),
    the down dgrad blocks W_down along d (its columns: exact here).  The
    same layer with the weight blockings swapped is not exact."""
    wl, x, dout, Wgu, Wd, rt = _mx_axis_case(33)
    Xp = O.dispatch(x, rt)
    segs = list(zip(rt["offsets"][:-1], rt["offsets"][1:]))
    H = np.concatenate([Xp[s0:s1] @ Wgu[e].T for e, (s0, s1) in enumerate(segs)])
    tok = rt["src_of"] // wl.k
    G = np.concatenate([dout[tok[s0:s1]] @ Wd[e] for e, (s0, s1) in enumerate(segs)])

    def run(recipe):
        f = O.forward_fp8(x, rt, Wgu, Wd, recipe=recipe)
        b = O.backward_fp8(dout, rt, Wgu, Wd, f, recipe=recipe)
        dw_row = np.sum(G * O.swiglu(f["H"], wl.I), axis=1)
        return f, b, dw_row[rt["row_of"]].reshape(wl.T, wl.k)
    f, b, dtw = run(O.MXFP8)
    assert np.array_equal(f["H"], O.bf16_round(H))
    np.testing.assert_allclose(b["d_topk_w"], dtw, rtol=1e-13, atol=1e-13 * np.max(np.abs(dtw)))
    f, b, dtw = run(dict(O.MXFP8, w_fwd=O.mx_cols, w_bwd=O.mx_rows))
    assert not np.array_equal(f["H"], O.bf16_round(H))
    assert not np.allclose(b["d_topk_w"], dtw, rtol=1e-6, atol=0)


def test_mx_layer_close_to_unquantised_layer():
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=256, T=64, dtype="bf16")
    inp = {k: _np(v) for k, v in S.make_inputs(wl, seed=15).items()}
    rt = O.route(inp["logits"], wl.k, wl.E)
    fw = O.forward(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    bw = O.backward(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], fw)
    fm = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"], recipe=O.MXFP8)
    bm = O.backward_fp8(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], fm, recipe=O.MXFP8)
    for ref, got in ((fw["out"], fm["out"]), (bw["dx"], bm["dx"]),
                     (bw["dW_gate_up"], bm["dW_gate_up"]), (bw["dW_down"], bm["dW_down"]),
                     (bw["d_topk_w"], bm["d_topk_w"])):
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        assert 1e-3 < err < 0.1


def test_mx_sampled_evaluators_match_full_layer():
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=128, T=96, E=6, k=2, dtype="bf16")
    inp = {k: _np(v) for k, v in S.make_inputs(wl, seed=34).items()}
    rt = O.route(inp["logits"], wl.k, wl.E)
    fm = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"], recipe=O.MXFP8)
    bm = O.backward_fp8(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], fm, logits=inp["logits"],
                        recipe=O.MXFP8)
    toks = np.array([0, 7, 60, 95])
    s = O.forward_backward_tokens_fp8(inp["x"], inp["logits"], inp["dout"], inp["w_gate_up"],
                                      inp["w_down"], wl.k, toks, recipe=O.MXFP8)
    for n, ref in (("out", fm["out"]), ("dx", bm["dx"]), ("d_topk_w", bm["d_topk_w"]),
                   ("dlogits", bm["dlogits"])):
        np.testing.assert_allclose(s[n], ref[toks], rtol=1e-12, atol=1e-12 * np.max(np.abs(ref)))
    for e in range(wl.E):
        dgu, dd = O.expert_weight_grads_fp8(inp["x"], inp["dout"], rt, inp["w_gate_up"], inp["w_down"],
                                            e, recipe=O.MXFP8)
        np.testing.assert_allclose(dgu, bm["dW_gate_up"][e], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dd, bm["dW_down"][e], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- fp8_bwd

def test_unquantised_recipe_is_the_bf16_storage_forward():
    """forward_fp8 with NO_QUANT: the exact forward with H and Aw rounded to
    bf16 once (H bit-equal to the rounded exact H, out within bf16 error)."""
    wl, inp = _tiny(seed=40, T=48, dtype="bf16")
    rt = O.route(inp["logits"], wl.k, wl.E)
    fw = O.forward(inp["x"], rt, inp["w_gate_up"], inp["w_down"])
    f0 = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"], recipe=O.NO_QUANT)
    assert np.array_equal(f0["H"], O.bf16_round(fw["H"]))
    w_row = rt["w"].ravel()[rt["src_of"]]
    assert np.array_equal(f0["Aw"], O.bf16_round(w_row[:, None] * fw["A"]))
    err = np.max(np.abs(f0["out"] - fw["out"])) / np.max(np.abs(fw["out"]))
    assert 0 < err < 2 ** -7


def test_fp8_bwd_sampled_evaluators_match_full_layer():
    wl = S.WORKLOADS["tiny"].scaled(d=256, I=128, T=96, E=6, k=2, dtype="bf16")
    inp = {k: _np(v) for k, v in S.make_inputs(wl, seed=41).items()}
    rt = O.route(inp["logits"], wl.k, wl.E)
    f0 = O.forward_fp8(inp["x"], rt, inp["w_gate_up"], inp["w_down"], recipe=O.NO_QUANT)
    b8 = O.backward_fp8(inp["dout"], rt, inp["w_gate_up"], inp["w_down"], f0, logits=inp["logits"])
    toks = np.array([0, 3, 47, 95])
    s = O.forward_backward_tokens_fp8(inp["x"], inp["logits"], inp["dout"], inp["w_gate_up"],
                                      inp["w_down"], wl.k, toks, fwd_recipe=O.NO_QUANT)
    for n, ref in (("out", f0["out"]), ("dx", b8["dx"]), ("d_topk_w", b8["d_topk_w"]),
                   ("dlogits", b8["dlogits"])):
        np.testing.assert_allclose(s[n], ref[toks], rtol=1e-12, atol=1e-12 * np.max(np.abs(ref)))
    for e in range(wl.E):
        dgu, dd = O.expert_weight_grads_fp8(inp["x"], inp["dout"], rt, inp["w_gate_up"], inp["w_down"],
                                            e, fwd_recipe=O.NO_QUANT)
        np.testing.assert_allclose(dgu, b8["dW_gate_up"][e], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dd, b8["dW_down"][e], rtol=1e-12, atol=1e-12)
