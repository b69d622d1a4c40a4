"""Pins of the clamped SwiGLU in the oracle.

The pages name DeepSeek V4's clamped SwiGLU (activations.ClampedSilu) as one
the layer takes and give neither its form nor its constant ("Mario/overlap
moe kernel integration", commit on ClampedSwiglu).  Reading, with the limit
L an argument: a = silu(min(g, L)) * clamp(u, -L, L), no gradient through an
active clamp.  The pins: a case worked by hand, finite differences of the
whole layer away from the clamp's kinks, torch's own clamp / silu / autograd
on a dense one-expert layer, the plain SwiGLU when no value reaches the
limit, and planted mistakes that these catch.  CPU only.
"""
import math

import numpy as np
import torch

from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O


def _tiny(seed, **kw):
    wl = S.WORKLOADS["tiny"].scaled(**kw)
    inp = S.make_inputs(wl, seed=seed)
    return wl, {k: v.double().numpy() for k, v in inp.items()}


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_hand_worked_clamped_example():
    """One token, one expert, d = 2, I = 2, L = 2: gate (3, -1), up (5, -0.5).
    The first gate and the first up value are clamped (to 2 and 2); the
    second pair passes unchanged."""
    x = np.array([[1.0, 0.0]])
    Wgu = np.array([[[3.0, 0.0], [-1.0, 0.0], [5.0, 0.0], [-0.5, 0.0]]])   # rows: g0 g1 u0 u1
    Wd = np.array([[[1.0, 1.0], [0.0, 1.0]]])
    rt = O.route(None, 1, 1, ids=np.zeros((1, 1), int), w=np.ones((1, 1)))
    f = O.forward(x, rt, Wgu, Wd, limit=2.0)
    a0 = 2.0 * _sig(2.0) * 2.0           # silu(min(3, 2)) * clamp(5)
    a1 = -1.0 * _sig(-1.0) * -0.5        # silu(-1) * (-0.5)
    np.testing.assert_allclose(f["A"][0], [a0, a1], rtol=1e-15)
    np.testing.assert_allclose(f["out"][0], [a0 + a1, a1], rtol=1e-15)
    # dout = (1, 0): dA = W_d^T dout = (1, 1)
    b = O.backward(np.array([[1.0, 0.0]]), rt, Wgu, Wd, f, limit=2.0)
    s1 = _sig(-1.0)
    dg1 = 1.0 * -0.5 * s1 * (1.0 + -1.0 * (1.0 - s1))   # gate -1: unclamped
    du1 = 1.0 * -1.0 * s1                                # up -0.5: unclamped
    # g0 = 3 and u0 = 5 sit above the limit: no gradient reaches them
    dH = np.array([0.0, dg1, 0.0, du1])
    np.testing.assert_allclose(b["dW_gate_up"][0][:, 0], dH, rtol=1e-15, atol=0)
    np.testing.assert_allclose(b["dx"][0], [dH @ Wgu[0][:, 0], 0.0], rtol=1e-15, atol=1e-300)


def _limit_away_from_kinks(H, I, lo, hi, gap):
    """A limit in [lo, hi] at least `gap` away from every gate value and
    every |up| value, so that finite differences never cross a kink."""
    vals = np.concatenate([H[:, :I].ravel(), np.abs(H[:, I:]).ravel()])
    for L in np.linspace(lo, hi, 2001):
        if np.min(np.abs(vals - L)) > gap:
            return float(L)
    raise AssertionError("no limit away from the kinks")


def _loss(x, rt, Wgu, Wd, dout, L):
    return float(np.sum(dout * O.forward(x, rt, Wgu, Wd, limit=L)["out"]))


def test_clamped_backward_finite_differences():
    wl, inp = _tiny(seed=21, T=32)
    x, lg, Wgu, Wd, dout = (inp[n] for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    rt = O.route(lg, wl.k, wl.E)
    H = O.forward(x, rt, Wgu, Wd)["H"]
    L = _limit_away_from_kinks(H, wl.I, 0.6, 0.9, 2e-4)
    gc = H[:, :wl.I] > L
    uc = np.abs(H[:, wl.I:]) > L
    assert 0.05 < gc.mean() < 0.75 and 0.05 < uc.mean() < 0.75   # both clamps are active somewhere
    fw = O.forward(x, rt, Wgu, Wd, limit=L)
    g = O.backward(dout, rt, Wgu, Wd, fw, logits=lg, limit=L)
    rng = np.random.default_rng(22)
    h = 1e-7
    for name, arr, grad in (("x", x, g["dx"]), ("Wgu", Wgu, g["dW_gate_up"]), ("Wd", Wd, g["dW_down"])):
        for _ in range(3):
            v = rng.standard_normal(arr.shape)
            args = dict(x=x, Wgu=Wgu, Wd=Wd)
            args[name] = arr + h * v
            lp = _loss(args["x"], rt, args["Wgu"], args["Wd"], dout, L)
            args[name] = arr - h * v
            lm = _loss(args["x"], rt, args["Wgu"], args["Wd"], dout, L)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grad * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    for t in range(0, wl.T, 7):
        for j in range(wl.k):
            wp = rt["w"].copy(); wp[t, j] += h
            wm = rt["w"].copy(); wm[t, j] -= h
            rp = O.route(None, wl.k, wl.E, ids=rt["ids"], w=wp)
            rm = O.route(None, wl.k, wl.E, ids=rt["ids"], w=wm)
            fd = (_loss(x, rp, Wgu, Wd, dout, L) - _loss(x, rm, Wgu, Wd, dout, L)) / (2 * h)
            assert abs(fd - g["d_topk_w"][t, j]) <= 1e-6 * max(1.0, abs(fd))


def test_clamped_single_expert_matches_torch_autograd():
    """E = 1, k = 1: the layer is a dense MLP; torch's clamp and silu with
    its autograd give the reference forward and gradients."""
    rng = np.random.default_rng(23)
    T, d, I, L = 40, 24, 16, 0.7
    x = rng.standard_normal((T, d))
    Wgu = rng.standard_normal((1, 2 * I, d)) / math.sqrt(d)
    Wd = rng.standard_normal((1, d, I)) / math.sqrt(I)
    dout = rng.standard_normal((T, d))
    rt = O.route(np.zeros((T, 1)), 1, 1)
    f = O.forward(x, rt, Wgu, Wd, limit=L)
    b = O.backward(dout, rt, Wgu, Wd, f, limit=L)
    xt = torch.tensor(x, requires_grad=True)
    W1 = torch.tensor(Wgu[0], requires_grad=True)
    W2 = torch.tensor(Wd[0], requires_grad=True)
    h = xt @ W1.T
    a = torch.nn.functional.silu(torch.clamp(h[:, :I], max=L)) * torch.clamp(h[:, I:], -L, L)
    out = a @ W2.T
    out.backward(torch.tensor(dout))
    assert (h[:, :I] > L).any() and (h[:, I:].abs() > L).any()
    np.testing.assert_allclose(f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dW_gate_up"][0], W1.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dW_down"][0], W2.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_limit_above_every_value_is_the_plain_swiglu():
    wl, inp = _tiny(seed=24, T=48)
    x, lg, Wgu, Wd, dout = (inp[n] for n in ("x", "logits", "w_gate_up", "w_down", "dout"))
    rt = O.route(lg, wl.k, wl.E)
    f0 = O.forward(x, rt, Wgu, Wd)
    L = float(np.max(np.abs(f0["H"]))) * 1.01
    f1 = O.forward(x, rt, Wgu, Wd, limit=L)
    b0 = O.backward(dout, rt, Wgu, Wd, f0, logits=lg)
    b1 = O.backward(dout, rt, Wgu, Wd, f1, logits=lg, limit=L)
    assert np.array_equal(f0["out"], f1["out"])
    for n in ("dx", "dW_gate_up", "dW_down", "d_topk_w", "dlogits"):
        assert np.array_equal(b0[n], b1[n]), n


def test_clamped_planted_mistakes_are_caught(monkeypatch):
    """Gradient passed through an active clamp, or the gate clamped from
    below as well, must fail the torch pin above."""
    real_bwd, real_fwd = O.swiglu_backward, O.swiglu

    def leaky(H, dA, I, limit=0.0):      # clamps the values but lets every gradient through
        g, u = np.minimum(H[:, :I], limit), np.clip(H[:, I:], -limit, limit)
        s = O.sigmoid(g)
        return np.concatenate([dA * u * s * (1.0 + g * (1.0 - s)), dA * g * s], axis=1)

    def both_sides(H, I, limit=0.0):
        return O.silu(np.clip(H[:, :I], -limit, limit)) * np.clip(H[:, I:], -limit, limit)

    for name, fn in (("swiglu_backward", leaky), ("swiglu", both_sides)):
        monkeypatch.setattr(O, name, fn)
        try:
            test_clamped_single_expert_matches_torch_autograd()
        except AssertionError:
            pass
        else:
            raise AssertionError(f"planted mistake in {name} not caught")
        monkeypatch.setattr(O, "swiglu_backward", real_bwd)
        monkeypatch.setattr(O, "swiglu", real_fwd)
