"""fp8 operand blockings of the HIP layer, held tightly to the oracle.

The layer tolerance for fp8 (6e-2) is loose enough that a GEMM quantising
one operand in the wrong blocks could pass it.  These two layers are built so
that it cannot: every value is an e4m3 number times a power of two, the block
scales come out as powers of two, each GEMM input is a single product or a
short sum that float32 holds exactly, and gate pre-activations of at least 256
make sigmoid(g) exactly 1 on both sides.  The GPU's H, Aw, G and dH then
equal the oracle's bit for bit, so both sides quantise identical values and
the results differ only by float32 accumulation order and bfloat16 storage:
the tolerance here is 1e-2 (the bf16 layer's is 2e-2), measured per token or
per block of equal binades so that small-binade parts are judged on their
own scale.

Binades differ by 2^20 along the axis a wrong blocking would mix:
* per token ("row" layer): the forward down GEMM's Aw, the down dgrad's dout
  and the gate/up dgrad's dH are blocked along K inside one token's row; in
  token runs they would mix tokens and flush the small ones;
* per column ("column" layer): both operands of each weight gradient are
  blocked in runs of one column; in rows they would mix columns.  dout and
  the gathered x take their binades from the inputs in both formats.  Aw and
  dH take theirs from the weights: per column in MXFP8, whose weight blocks
  run along one axis only, and per 128-column group in blockwise FP8, whose
  128 x 128 weight blocks would flush a finer pattern.  The two formats share
  one operand wiring in the backward (the quantiser launches take a format
  flag), so the MXFP8 case covers the wiring of both.

Each case first checks on the CPU that the oracle with the one operand's
blocking swapped misses the tolerance by far (a planted mistake in a copy of
the oracle), then runs the GPU.
"""
import numpy as np
import pytest
import torch

from combine_top_route_amd import synthetic as S
from oracle import moe_oracle as O

from gpu_util import check_routing, run_gpu, run_oracle
from test_oracle_fp8_blockings import _mutant

pytestmark = pytest.mark.gpu

T, E, K, D, I = 600, 3, 2, 256, 256          # every expert: 400 rows (three 128-row runs and a short one)
GRID = np.array([8, 9, 10, 11, 12, 13], dtype=np.float64) * 32.0   # e4m3 values 256..416
MARK = 448.0
TOL = 1e-2
RECIPES = {"fp8_block": O.FP8_BLOCK, "mxfp8": O.MXFP8}


def _routing():
    t = np.arange(T)
    ids = np.stack([t % E, (t + 1) % E], axis=1).astype(np.int32)
    return torch.from_numpy(ids), torch.full((T, K), 0.5, dtype=torch.float32)


def _grid(rng, shape):
    return rng.choice(GRID, shape) * rng.choice([-1.0, 1.0], shape)


def _sign(rng, shape):
    return rng.choice([-1.0, 1.0], shape)


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.double().numpy(), a), "construction must be bf16-exact"
    return t


def _row_layer(rng):
    """Per-token binades: a (x, 2^0 or 2^20) and b (dout, 2^0 or 2^-20)."""
    a = rng.choice([0, 20], T)
    b = rng.choice([0, -20], T)
    x = np.zeros((T, D))
    x[:, 0] = MARK * 2.0 ** a                # row-block mark; W_gate_up column 0 is zero
    x[:, 1] = 256.0 * 2.0 ** a               # the value the gate/up GEMM uses
    Wgu = np.zeros((E, 2 * I, D))
    Wgu[:, :I, 1] = 256.0 * 2.0 ** -8        # g = 2^(8 + a)
    Wgu[:, I:, 1] = _grid(rng, (E, I)) * 2.0 ** -8
    Wgu[:, I::128, 1] = MARK * _sign(rng, (E, I // 128)) * 2.0 ** -8
    Wgu[:, :, 2] = MARK * 2.0 ** -8          # weight-block marks (x column 2 is zero)
    Wd = _grid(rng, (E, D, I))
    Wd[:, ::128, ::128] = MARK * _sign(rng, (E, D // 128, I // 128))
    Wd *= 2.0 ** -6
    dout = np.zeros((T, D))
    dout[:, 0] = MARK * _sign(rng, T) * 2.0 ** b
    return x, Wgu, Wd, dout


def _column_layer(rng, mx):
    """Per-column binades: beta (x columns), delta (dout columns), gamma (the
    up rows of W_gate_up, hence Aw's columns), omega (W_down's columns, hence
    G's and dH's columns); gamma and omega per 128-column group unless mx."""
    def per(n):
        v = rng.choice([0, -20], n)
        if not mx:
            v = np.repeat(rng.choice([0, -20], n // 128), 128)
        return v
    beta, delta = rng.choice([0, -20], D), rng.choice([0, -20], D)
    gamma, omega = per(I), per(I)
    beta[:3] = delta[:3] = 0
    x = _grid(rng, (T, D)) * 2.0 ** beta
    x[:, 0] = rng.choice(GRID, T)            # m_t > 0: g = m_t W_gate[i, 0] >= 256
    x[:, 1] = MARK                           # row-block mark
    x[:, 2] = 0.0                            # the weights' mark column
    Wgu = np.zeros((E, 2 * I, D))
    Wgu[:, :I, 0] = rng.choice(GRID, (E, I)) * 2.0 ** -8
    Wgu[:, I:, 0] = _grid(rng, (E, I)) * 2.0 ** (gamma - 8)
    Wgu[:, :, 2] = MARK * 2.0 ** (np.concatenate([np.zeros(I), gamma]) - 8)
    Wd = np.zeros((E, D, I))
    Wd[:, 0, :] = _grid(rng, (E, I)) * 2.0 ** (omega - 6)
    Wd[:, 1, :] = MARK * 2.0 ** (omega - 6)
    dout = _grid(rng, (T, D)) * 2.0 ** delta
    dout[:, 0] = rng.choice(GRID, T) * _sign(rng, T)
    dout[:, 1] = MARK
    dout[:, 2] = 0.0
    cls = dict(x=beta, dout=delta, aw=gamma, dh=np.concatenate([omega + gamma, omega]))
    return x, Wgu, Wd, dout, cls


def _inputs(x, Wgu, Wd, dout):
    return {"x": _bf16(x), "w_gate_up": _bf16(Wgu), "w_down": _bf16(Wd), "dout": _bf16(dout),
            "logits": torch.zeros((T, E), dtype=torch.bfloat16)}


def _per_row_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=1)
    err = np.max(np.abs(got - ref), axis=1)
    assert np.all(err[den == 0] == 0)
    nz = den > 0
    return float(np.max(err[nz] / den[nz]))


def _class_err(got, ref, rcls, ccls):
    """Largest max|err| / max|ref| over the blocks of rows of one class by
    columns of one class."""
    worst = 0.0
    for a in np.unique(rcls):
        for b in np.unique(ccls):
            g = got[np.ix_(rcls == a, ccls == b)]
            r = ref[np.ix_(rcls == a, ccls == b)]
            den = np.max(np.abs(r))
            if den == 0:
                assert np.all(g == 0)
                continue
            worst = max(worst, float(np.max(np.abs(g - r)) / den))
    return worst


def _oracle(fwd, bwd, wl, inp, ids, w, recipe):
    rt = O.route(None, wl.k, wl.E, ids=ids.numpy(), w=w.double().numpy())
    f = lambda t: t.double().numpy()
    Wgu, Wd = inp["w_gate_up"].float().numpy(), inp["w_down"].float().numpy()
    fw = fwd(f(inp["x"]), rt, Wgu, Wd, recipe=recipe)
    res = dict(fw)
    res.update(bwd(f(inp["dout"]), rt, Wgu, Wd, fw, recipe=recipe))
    return res


def _workload(name):
    return S.WORKLOADS["tiny"].scaled(T=T, d=D, E=E, k=K, I=I, dtype="bf16", logits_dtype="bf16",
                                      precision=name)


def _row_metrics(res):
    return {n: res[n] for n in ("out", "dx", "d_topk_w")}


@pytest.mark.parametrize("name", list(RECIPES))
def test_fp8_row_blockings_tight(name):
    recipe = RECIPES[name]
    wl = _workload(name)
    ids, w = _routing()
    inp = _inputs(*_row_layer(np.random.default_rng(11)))
    ref = _oracle(O.forward_fp8, O.backward_fp8, wl, inp, ids, w, recipe)
    # planted mistakes (CPU): each row-blocked operand in token runs instead
    mistakes = {
        "Aw (forward down)": (_mutant(O.forward_fp8, 'recipe["act"](Aw[s])', 'recipe["tok"](Aw[s])'),
                              O.backward_fp8, "out"),
        "dout (down dgrad)": (O.forward_fp8, _mutant(O.backward_fp8, 'recipe["act"](dout[tok[s]]) @ Wd_q',
                                                     'recipe["tok"](dout[tok[s]]) @ Wd_q'), "d_topk_w"),
        "dH (gate/up dgrad)": (O.forward_fp8, _mutant(O.backward_fp8, 'recipe["act"](dH) @ Wgu_q',
                                                      'recipe["tok"](dH) @ Wgu_q'), "dx"),
    }
    for what, (fwd, bwd, out) in mistakes.items():
        bad = _oracle(fwd, bwd, wl, inp, ids, w, recipe)
        assert _per_row_err(bad[out], ref[out]) > 0.5, what
    print(f"case fp8 row blockings {name}: T={T} d={D} I={I} E={E} k={K}", flush=True)
    gpu = run_gpu(wl, inp, ids=ids, w=w)
    check_routing(gpu, {"rt": O.route(None, K, E, ids=ids.numpy(), w=w.double().numpy())})
    errs = {n: _per_row_err(gpu[n], ref[n]) for n in ("out", "dx", "d_topk_w")}
    print(name, errs)
    assert all(e <= TOL for e in errs.values()), errs


@pytest.mark.parametrize("name", list(RECIPES))
def test_fp8_weight_gradient_blockings_tight(name):
    recipe = RECIPES[name]
    mx = name == "mxfp8"
    wl = _workload(name)
    ids, w = _routing()
    x, Wgu, Wd, dout, cls = _column_layer(np.random.default_rng(12), mx)
    inp = _inputs(x, Wgu, Wd, dout)
    ref = _oracle(O.forward_fp8, O.backward_fp8, wl, inp, ids, w, recipe)

    def errs(res):
        e_d = max(_class_err(res["dW_down"][e], ref["dW_down"][e], cls["dout"], cls["aw"]) for e in range(E))
        e_g = max(_class_err(res["dW_gate_up"][e], ref["dW_gate_up"][e], cls["dh"], cls["x"]) for e in range(E))
        return {"dW_down": e_d, "dW_gate_up": e_g}
    # planted mistakes (CPU): a weight-gradient operand in rows instead of token runs
    swaps = {"dout": ('recipe["tok"](dout[tok[s]])', 'recipe["act"](dout[tok[s]])', "dW_down"),
             "x": ('recipe["tok"](Xp[s])', 'recipe["act"](Xp[s])', "dW_gate_up")}
    if mx:
        swaps.update({"Aw": ('recipe["tok"](Aw[s])', 'recipe["act"](Aw[s])', "dW_down"),
                      "dH": ('recipe["tok"](dH).T', 'recipe["act"](dH).T', "dW_gate_up")})
    for what, (old, new, out) in swaps.items():
        bad = _oracle(O.forward_fp8, _mutant(O.backward_fp8, old, new), wl, inp, ids, w, recipe)
        assert errs(bad)[out] > 0.5, what
    print(f"case fp8 weight-gradient blockings {name}: T={T} d={D} I={I} E={E} k={K}", flush=True)
    gpu = run_gpu(wl, inp, ids=ids, w=w)
    e = errs(gpu)
    rest = {n: _per_row_err(gpu[n], ref[n]) for n in ("out", "dx", "d_topk_w")}
    print(name, e, rest)
    assert all(v <= TOL for v in e.values()), e
    assert all(v <= TOL for v in rest.values()), rest
