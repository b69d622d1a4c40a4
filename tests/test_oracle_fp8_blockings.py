"""Pins of the fp8 oracle's operand blockings, GEMM by GEMM.

Blockwise FP8 shares one scale over a block of values ("Prime Intellect's
Prime Mega MoE Trains Giant AI Models 55% Faster", section "Precision and
hardware support"); the blocks each GEMM operand takes are readings (1 x 128
rows along K for activations and gradients, 128 x 128 for weights, 128-token
runs from each expert's first row for both weight-gradient operands; MXFP8:
the same with 32-value blocks and power-of-two scales).

Each pin builds operands that sit exactly on the e4m3 grid of the blocking
the reading gives one GEMM: every value is an e4m3 number times a power of
two that is constant inside each intended block, and every blockwise block
holds one value of magnitude 448 * 2^s, so its scale is exactly 2^s.  The
power of two changes by 2^20 across the other axis, so any block that runs
along that axis mixes binades and cannot be exact.  Quantisation under the
intended blocking is then the identity and the GEMM equals the unquantised
product computed from the same arrays; under a swapped blocking it does not.
Each pin is also run against a copy of the oracle with that one operand's
blocking swapped, which must fail it (a planted mistake, on the CPU).

Internal operands are controlled without a special entry point: the backward
takes the forward's H, Aw and Xp as inputs, and gate pre-activations of at
least 64 make sigmoid(g) exactly 1 in float64, so the SwiGLU backward is
dg = dA * up and du = dA * g and the gradient dH stays on the grid.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import moe_oracle as O

T, E, K, D, I = 300, 3, 2, 256, 128
GRID = np.array([8, 9, 10, 11, 12, 13], dtype=np.float64) * 32.0   # e4m3 values 256..416
MARK = 448.0
LO = -20                                                              # the other binade

RECIPES = {"fp8_block": O.FP8_BLOCK, "mxfp8": O.MXFP8}


def _routing():
    # every expert gets 200 rows: one full 128-row run and a ragged one
    t = np.arange(T)
    ids = np.stack([t % E, (t + 1) % E], axis=1)
    rt = O.route(None, K, E, ids=ids, w=np.full((T, K), 0.5))
    assert np.all(rt["counts"] == 200)
    return rt


def _grid(rng, shape):
    return rng.choice(GRID, shape) * rng.choice([-1.0, 1.0], shape)


def _sign(rng, shape):
    return rng.choice([-1.0, 1.0], shape)


def _run_starts(rt):
    """Expert-sorted rows that open a 128-row token run of their expert."""
    off = rt["offsets"]
    return np.concatenate([np.arange(off[e], off[e + 1], 128) for e in range(E)])


def _weights(rng, n, k, q=-6):
    """[E, n, k] weights exact under 128 x 128 blocks (a 448 at each block's
    corner, every other magnitude below 448) and under any MXFP8 blocking
    (one binade per expert, every magnitude in (224, 448])."""
    W = _grid(rng, (E, n, k))
    W[:, ::128, ::128] = MARK * _sign(rng, W[:, ::128, ::128].shape)
    return W * 2.0 ** q


def _segments(rt):
    off = rt["offsets"]
    return [slice(off[e], off[e + 1]) for e in range(E)]


def _close(got, ref, ref_abs):
    """Equal up to float64 rounding of the product (bounded by the product
    of absolute values)."""
    return bool(np.all(np.abs(got - ref) <= 1e-12 * ref_abs))


def _mutant(fn, old, new):
    """A copy of an oracle function with one expression replaced."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, (fn.__name__, old)
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    return ns[fn.__name__]


# ---------------------------------------------------------------- forward down GEMM: Aw in 1 x K rows

def _case_fwd_down(rng):
    rt = _routing()
    a = rng.choice([0, 20], T)                       # one binade per token
    x = np.zeros((T, D))
    x[:, 0] = MARK * 2.0 ** a                        # block mark (column 0 of W_gate_up is zero)
    x[:, 1] = 256.0 * 2.0 ** a                       # the value the GEMM uses
    Wgu = np.zeros((E, 2 * I, D))
    Wgu[:, :I, 1] = 256.0 * 2.0 ** -8                # gate = 2^(8 + a): sigmoid(g) == 1
    Wgu[:, I:, 1] = _grid(rng, (E, I))
    Wgu[:, I::128, 1] = MARK * _sign(rng, (E, 1))    # each 128 block of up holds a 448
    Wgu[:, :, 2] = MARK * np.where(np.arange(2 * I) < I, 2.0 ** -8, 1.0)   # weight block marks
    Wd = _weights(rng, D, I)
    return rt, x, Wgu, Wd


def _pin_fwd_down(forward, recipe, rng):
    rt, x, Wgu, Wd = _case_fwd_down(rng)
    f = forward(x, rt, Wgu, Wd, recipe=recipe)
    # the SwiGLU output is a power of two times a grid value: stored exactly
    g, u = f["H"][:, :I], f["H"][:, I:]
    assert np.all(g >= 256) and np.array_equal(f["Aw"], 0.5 * g * u)
    ok = True
    for e, s in enumerate(_segments(rt)):
        ref = f["Aw"][s] @ Wd[e].T
        ok &= _close(f["Yw"][s], ref, np.abs(f["Aw"][s]) @ np.abs(Wd[e]).T)
    return ok


@pytest.mark.parametrize("name", list(RECIPES))
def test_forward_down_gemm_blocks_aw_along_rows(name):
    recipe = RECIPES[name]
    assert _pin_fwd_down(O.forward_fp8, recipe, np.random.default_rng(1))
    bad = _mutant(O.forward_fp8, 'recipe["act"](Aw[s])', 'recipe["tok"](Aw[s])')
    assert not _pin_fwd_down(bad, recipe, np.random.default_rng(1))
    if name == "fp8_block":   # the down weight in 128 x 128 blocks, not in rows
        assert not _pin_fwd_down(O.forward_fp8, dict(recipe, w_fwd=O.quant_rows_1x128),
                                 np.random.default_rng(1))


# ---------------------------------------------------------------- backward: injected forward tensors

def _bwd(backward, dout, rt, Wgu, Wd, H, Aw, Xp, recipe):
    fwd = dict(H=H, Aw=Aw, Xp=Xp)
    return backward(dout, rt, Wgu, Wd, fwd, recipe=recipe)


def _case_down_dgrad(rng):
    rt = _routing()
    p = rng.choice([0, LO], T)                       # one binade per token
    dout = _grid(rng, (T, D)) * 2.0 ** p[:, None]
    dout[:, ::128] = MARK * _sign(rng, (T, D // 128)) * 2.0 ** p[:, None]
    Wd = _weights(rng, D, I)
    Wgu = _weights(rng, 2 * I, D)
    R = T * K
    H = rng.standard_normal((R, 2 * I))
    return rt, dout, Wgu, Wd, H, np.zeros((R, I)), np.zeros((R, D))


def _pin_down_dgrad(backward, recipe, rng):
    """Down dgrad G = dout W_down[e] (dout in 1 x 128 rows along d, W_down in
    weight blocks): seen through the top-k-weight gradient <G, a>."""
    rt, dout, Wgu, Wd, H, Aw, Xp = _case_down_dgrad(rng)
    b = _bwd(backward, dout, rt, Wgu, Wd, H, Aw, Xp, recipe)
    tok = rt["src_of"] // K
    R = T * K
    ref, ref_abs = np.zeros(R), np.zeros(R)
    for e, s in enumerate(_segments(rt)):
        a = O.swiglu(H[s], I)
        ref[s] = np.sum((dout[tok[s]] @ Wd[e]) * a, axis=1)
        ref_abs[s] = np.sum((np.abs(dout[tok[s]]) @ np.abs(Wd[e])) * np.abs(a), axis=1)
    got = b["d_topk_w"].ravel()[rt["src_of"]]
    return _close(got, ref, ref_abs)


@pytest.mark.parametrize("name", list(RECIPES))
def test_down_dgrad_blocks_dout_along_rows(name):
    recipe = RECIPES[name]
    assert _pin_down_dgrad(O.backward_fp8, recipe, np.random.default_rng(2))
    bad = _mutant(O.backward_fp8, 'recipe["act"](dout[tok[s]]) @ Wd_q', 'recipe["tok"](dout[tok[s]]) @ Wd_q')
    assert not _pin_down_dgrad(bad, recipe, np.random.default_rng(2))
    if name == "fp8_block":
        assert not _pin_down_dgrad(O.backward_fp8, dict(recipe, w_bwd=O.quant_rows_1x128),
                                   np.random.default_rng(2))


def _case_down_wgrad(rng):
    rt = _routing()
    beta = rng.choice([0, LO], D)                    # one binade per column of dout
    gamma = rng.choice([0, LO], I)                   # and per column of Aw
    dout = _grid(rng, (T, D)) * 2.0 ** beta
    tok = rt["src_of"] // K
    runs = _run_starts(rt)
    dout[tok[runs]] = MARK * _sign(rng, (runs.size, D)) * 2.0 ** beta
    R = T * K
    Aw = _grid(rng, (R, I)) * 2.0 ** gamma
    Aw[runs] = MARK * _sign(rng, (runs.size, I)) * 2.0 ** gamma
    H = rng.standard_normal((R, 2 * I))
    return rt, dout, _weights(rng, 2 * I, D), _weights(rng, D, I), H, Aw, np.zeros((R, D))


def _pin_down_wgrad(backward, recipe, rng):
    """Down wgrad dW_down[e] = dout^T Aw over the expert's rows, both in
    token runs counted from the expert's first row."""
    rt, dout, Wgu, Wd, H, Aw, Xp = _case_down_wgrad(rng)
    b = _bwd(backward, dout, rt, Wgu, Wd, H, Aw, Xp, recipe)
    tok = rt["src_of"] // K
    ok = True
    for e, s in enumerate(_segments(rt)):
        ref = dout[tok[s]].T @ Aw[s]
        ok &= _close(b["dW_down"][e], ref, np.abs(dout[tok[s]]).T @ np.abs(Aw[s]))
    return ok


@pytest.mark.parametrize("name", list(RECIPES))
def test_down_wgrad_blocks_both_operands_in_token_runs(name):
    recipe = RECIPES[name]
    assert _pin_down_wgrad(O.backward_fp8, recipe, np.random.default_rng(3))
    # dout or Aw in 1 x 128 row blocks (the mistake that a 6e-2 layer
    # tolerance cannot see) must fail
    for old, new in (('recipe["tok"](dout[tok[s]])', 'recipe["act"](dout[tok[s]])'),
                     ('recipe["tok"](Aw[s])', 'recipe["act"](Aw[s])')):
        bad = _mutant(O.backward_fp8, old, new)
        assert not _pin_down_wgrad(bad, recipe, np.random.default_rng(3)), old


def _case_gateup(rng, per_token):
    """dout one-hot in column 0 (448 * 2^p), W_down nonzero in rows 0 (a power
    of two) and 1 (the block mark) only, so G = dout W_down[e] is 7 * 2^j
    (448 times a power of two) everywhere.  H = [g, u] with g a power of two
    of at least 64 and u = +-2^eta: dH = [w G u, w G g] holds magnitudes
    448 * 2^s only.  per_token: the binade varies by token (p), constant
    along each row; else by column (eta, zeta), constant down each column."""
    rt = _routing()
    R = T * K
    p = rng.choice([0, LO], T) if per_token else np.zeros(T, dtype=int)
    dout = np.zeros((T, D))
    dout[:, 0] = MARK * _sign(rng, T) * 2.0 ** p
    Wd = np.zeros((E, D, I))
    Wd[:, 0, :] = 256.0 * _sign(rng, (E, I)) * 2.0 ** -6
    Wd[:, 1, :] = MARK * _sign(rng, (E, I)) * 2.0 ** -6
    if per_token:
        eta, zeta = np.zeros(I), np.full(I, 6)
    else:
        eta, zeta = rng.choice([0, LO], I), rng.choice([6, 26], I)
    H = np.concatenate([np.broadcast_to(2.0 ** zeta, (R, I)),
                        _sign(rng, (R, I)) * 2.0 ** eta], axis=1)
    return rt, dout, Wd, H


def _dH_exact(rt, dout, Wd, H):
    """dH of this construction: sigmoid(g) == 1, so dg = w G u, du = w G g."""
    tok = rt["src_of"] // K
    dH = np.zeros((T * K, 2 * I))
    for e, s in enumerate(_segments(rt)):
        G = dout[tok[s]] @ Wd[e]
        dH[s] = np.concatenate([0.5 * G * H[s, I:], 0.5 * G * H[s, :I]], axis=1)
    return dH


def _pin_gateup_dgrad(backward, recipe, rng):
    """Gate/up dgrad dXp = dH W_gate_up[e] (dH in 1 x 128 rows along 2I),
    seen through dx = sum over a token's rows."""
    rt, dout, Wd, H = _case_gateup(rng, per_token=True)
    Wgu = _weights(rng, 2 * I, D)
    R = T * K
    b = _bwd(backward, dout, rt, Wgu, Wd, H, np.zeros((R, I)), np.zeros((R, D)), recipe)
    dH = _dH_exact(rt, dout, Wd, H)
    assert np.all(np.isin(np.abs(dH) / 2.0 ** np.floor(np.log2(np.abs(dH))), [1.75]))
    dXp, dXp_abs = np.zeros((R, D)), np.zeros((R, D))
    for e, s in enumerate(_segments(rt)):
        dXp[s] = dH[s] @ Wgu[e]
        dXp_abs[s] = np.abs(dH[s]) @ np.abs(Wgu[e])
    ro = rt["row_of"].reshape(T, K)
    ref = sum(dXp[ro[:, j]] for j in range(K))
    ref_abs = sum(dXp_abs[ro[:, j]] for j in range(K))
    return _close(b["dx"], ref, ref_abs)


@pytest.mark.parametrize("name", list(RECIPES))
def test_gateup_dgrad_blocks_dh_along_rows(name):
    recipe = RECIPES[name]
    assert _pin_gateup_dgrad(O.backward_fp8, recipe, np.random.default_rng(4))
    bad = _mutant(O.backward_fp8, 'recipe["act"](dH) @ Wgu_q', 'recipe["tok"](dH) @ Wgu_q')
    assert not _pin_gateup_dgrad(bad, recipe, np.random.default_rng(4))
    if name == "fp8_block":
        assert not _pin_gateup_dgrad(O.backward_fp8, dict(recipe, w_bwd=O.quant_rows_1x128),
                                     np.random.default_rng(4))


def _pin_gateup_wgrad(backward, recipe, rng):
    """Gate/up wgrad dW_gate_up[e] = dH^T Xp over the expert's rows, both in
    token runs counted from the expert's first row."""
    rt, dout, Wd, H = _case_gateup(rng, per_token=False)
    R = T * K
    beta = rng.choice([0, LO], D)
    Xp = _grid(rng, (R, D)) * 2.0 ** beta
    runs = _run_starts(rt)
    Xp[runs] = MARK * _sign(rng, (runs.size, D)) * 2.0 ** beta
    b = _bwd(backward, dout, rt, _weights(rng, 2 * I, D), Wd, H, np.zeros((R, I)), Xp, recipe)
    dH = _dH_exact(rt, dout, Wd, H)
    ok = True
    for e, s in enumerate(_segments(rt)):
        ref = dH[s].T @ Xp[s]
        ok &= _close(b["dW_gate_up"][e], ref, np.abs(dH[s]).T @ np.abs(Xp[s]))
    return ok


@pytest.mark.parametrize("name", list(RECIPES))
def test_gateup_wgrad_blocks_both_operands_in_token_runs(name):
    recipe = RECIPES[name]
    assert _pin_gateup_wgrad(O.backward_fp8, recipe, np.random.default_rng(5))
    for old, new in (('recipe["tok"](dH).T', 'recipe["act"](dH).T'),
                     ('recipe["tok"](Xp[s])', 'recipe["act"](Xp[s])')):
        bad = _mutant(O.backward_fp8, old, new)
        assert not _pin_gateup_wgrad(bad, recipe, np.random.default_rng(5)), old


def test_token_runs_are_counted_from_each_expert_first_row():
    """Blockwise token runs aligned to the expert's first row: with runs
    counted from row 0 of the sorted rows instead, the down wgrad's marked
    rows no longer open a run, and the pin fails."""
    shifted = dict(O.FP8_BLOCK)

    def tok_global(X, _q=O.quant_tokens_128):
        # a run boundary 64 rows into the segment stands in for a global alignment
        X = np.asarray(X)
        out = np.zeros(X.shape)
        out[:64] = _q(X[:64])
        out[64:] = _q(X[64:])
        return out
    shifted["tok"] = tok_global
    assert _pin_down_wgrad(O.backward_fp8, O.FP8_BLOCK, np.random.default_rng(3))
    assert not _pin_down_wgrad(O.backward_fp8, shifted, np.random.default_rng(3))
