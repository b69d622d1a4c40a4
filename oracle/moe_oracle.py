"""CPU oracle of the fused mixture-of-experts layer, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path: it is plain numpy in float64, written from the pages that
describe the method, step by step and in their order, without blocking or
fusion, so a reader can check it against those pages by eye.

Pages cited (title, then section):
  [P1] "Prime Intellect added the missing backward pass to DeepSeek's fused
       MoE kernel, making it usable for training ..." (AspireAI story)
  [P2] "Prime Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster"
       (alphasignal), sections "Where MoE training loses time",
       "One kernel overlaps the pipeline", "Precision and hardware support"
  [P3] "Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed"
       (phantom-byte), section "What a mixture-of-experts layer actually does"
  [P4] "Mario/overlap moe kernel integration" (prime-rl pull request 3651),
       overview and commit messages

What the pages fix, and the readings taken where they leave a step open:
  * routing: the router sends each token to a small subset of experts, top-8
    in the measured models [P2 "Where MoE training loses time"]; the routing
    tensors are per-token top scores and selected expert indices, plus the
    per-expert token counts [P4 commit "GroupedExperts.forward(x, *routing)"].
    Reading: the k experts with the largest logits, ties to the lower expert
    index; weights = softmax over the k selected logits (the same as a full
    softmax renormalised over the top k).
  * dispatch is "token sorting" into expert order [P2 "Where MoE training
    loses time"].  Reading: a stable sort of the flat (token, slot) entries by
    expert, so rows run expert-ascending, then token-ascending.
  * each expert is a two-layer MLP with SwiGLU [P3 "What a mixture-of-experts
    layer actually does"; P4 overview "SwiGLU expert GEMMs"].  Reading:
    W_gate_up[e] rows [0, I) are the gate, rows [I, 2I) the up projection;
    A = silu(gate) * up.  The pages also name DeepSeek V4's clamped SwiGLU
    (activations.ClampedSilu) as one the layer takes, and reject a
    differently defined ClampedSwiglu (sigmoid of 1.702 gate, up + 1) [P4
    commit on ClampedSwiglu]; they give neither the clamped form nor its
    constant.  Reading, with the constant an argument (limit > 0):
    A = silu(min(gate, limit)) * clamp(up, -limit, limit), no gradient
    through an active clamp.
  * combine returns expert outputs to their original positions [P2 "Where MoE
    training loses time"], summed with the top-k weights.
  * the backward repeats the exchange for gradients [P2 "Where MoE training
    loses time"; P1]; here it is the exact gradient of L = sum(dout * out)
    with respect to x, both weight tensors, the top-k weights and, through
    the renormalised softmax, the router logits (routing itself is piecewise
    constant and passes no gradient).
  * blockwise FP8 shares one scale over a block of values [P2 "Precision and
    hardware support"]; the workload fixes e4m3 with 1x128 activation blocks
    and 128x128 weight blocks.  Readings: scale = amax/448 in fp32 (1 where a
    block is all zero), round-to-nearest-even with saturation at +-448,
    weight-gradient GEMMs quantise both operands in 128-row blocks along the
    token dimension aligned to each expert's first row, the top-k weight is
    folded into the SwiGLU output before the down GEMM (Aw = w * a, which the
    down GEMM and the down wgrad quantise), the down dgrad quantises the
    unweighted upstream gradient, the top-k-weight gradient uses that
    dgrad's output, and the stored intermediates H, Aw and dH are bf16.
  * MXFP8 uses smaller scaling groups than blockwise FP8 [P2 "Precision and
    hardware support"] and is one of the layer's precision options [P4
    overview].  Reading: the OCP microscaling format MXFP8 -- blocks of 32
    values along each GEMM operand's contraction dimension, one power-of-two
    (E8M0) scale 2^X per block, elements rounded to nearest e4m3, ties to
    even.  The pages do not say how X is chosen; here it is the blockwise
    scale amax/448 rounded up to a power of two (the smallest X with amax <=
    448 * 2^X), so no value saturates, X >= -127 and X = 0 for an all-zero
    block.  The weights therefore take two blockings:
    along K for the forward GEMMs and along N for the data gradients; the
    weight-gradient operands take 32-token blocks from each expert's first
    row.  Everything else follows the blockwise FP8 readings above.
  * fp8_bwd is another of the layer's precision options [P4 overview], not
    described further.  Reading: FP8 in the backward only -- the forward of
    the bf16 layer (H and Aw stored in bf16) and the blockwise FP8 backward
    on those stored tensors: forward_fp8 with NO_QUANT, then backward_fp8
    with FP8_BLOCK.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# Routing  [P2 "Where MoE training loses time"; P4 commit on GroupedExperts]
# --------------------------------------------------------------------------

def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logit, largest first; among
    equal logits the lower expert index comes first.  Returns int64 [T, k]."""
    l = np.array(logits, dtype=F64)            # exact upcast
    T, E = l.shape
    taken = np.zeros((T, E), dtype=bool)
    ids = np.empty((T, k), dtype=np.int64)
    for j in range(k):
        masked = np.where(taken, -np.inf, l)
        # argmax returns the first index of the maximum: ties -> lower index.
        # -0.0 and +0.0 compare equal, so they tie as well.
        pick = np.argmax(masked, axis=1)
        # an expert already taken can only win again if every remaining logit
        # is -inf; then take the lowest untaken index (same tie rule).
        dup = taken[np.arange(T), pick]
        if dup.any():
            pick[dup] = np.argmax(~taken[dup], axis=1)
        ids[:, j] = pick
        taken[np.arange(T), pick] = True
    return ids


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w_tj = exp(l_tj) / sum_{i in S_t} exp(l_ti): softmax over the selected
    logits (float64 [T, k])."""
    l = np.array(logits, dtype=F64)
    sel = np.take_along_axis(l, ids, axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


def expert_counts(ids: np.ndarray, E: int):
    """counts[e] = number of (token, slot) entries routed to e;
    offsets = exclusive prefix sum, offsets[E] = T*k."""
    counts = np.zeros(E, dtype=np.int64)
    for e in ids.ravel():
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def expert_counts_fast(ids: np.ndarray, E: int):
    """Same as expert_counts, vectorised for large inputs."""
    counts = np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def token_sort(ids: np.ndarray, E: int):
    """Dispatch order: rows grouped by expert (ascending), and within an
    expert by flat entry f = t*k + j (ascending).

    Returns src_of [R] (row -> flat entry) and row_of [R] (flat entry -> row).
    """
    flat = np.asarray(ids).ravel()
    src_of = np.concatenate([np.nonzero(flat == e)[0] for e in range(E)]).astype(np.int64)
    row_of = np.empty_like(src_of)
    row_of[src_of] = np.arange(src_of.size)
    return src_of, row_of


def route(logits: np.ndarray | None, k: int, E: int,
          ids: np.ndarray | None = None, w: np.ndarray | None = None) -> dict:
    """All routing artefacts.  With logits=None, ids and w are taken as given
    (the "top_scores, selected_experts_indices" form)."""
    if logits is not None:
        ids = topk_select(logits, k)
        w = topk_weights(logits, ids)
    else:
        ids = np.asarray(ids, dtype=np.int64)
        w = np.asarray(w, dtype=F64)
    counts, offsets = expert_counts_fast(ids, E)
    src_of, row_of = token_sort(ids, E)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets,
                src_of=src_of, row_of=row_of, k=k, E=E)


# --------------------------------------------------------------------------
# Expert MLP  [P3 "What a mixture-of-experts layer actually does"]
# --------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu(H: np.ndarray, I: int, limit: float = 0.0) -> np.ndarray:
    """A = silu(gate) * up with gate = H[:, :I], up = H[:, I:].

    limit > 0: the clamped SwiGLU that the pages name for DeepSeek V4 (the
    PR's commit on activations.ClampedSilu), whose form and constant they
    do not give.  Reading: the gate is clamped from above and the up
    projection to [-limit, limit] before the product,
    A = silu(min(gate, limit)) * clamp(up, -limit, limit); the pages' other
    clamped variant (sigmoid of 1.702 gate, up + 1) is the one the kernel
    does not compute."""
    g, u = H[:, :I], H[:, I:]
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return silu(g) * u


def swiglu_backward(H: np.ndarray, dA: np.ndarray, I: int, limit: float = 0.0) -> np.ndarray:
    """d/dgate = dA * up * s(g) * (1 + g (1 - s(g))), d/dup = dA * silu(g).
    Clamped (limit > 0): g and up as clamped in the forward, and no gradient
    through a clamp that is active (gate above limit, |up| above limit); at
    the limit itself the gradient passes, as a clamp's derivative is taken
    one-sided from inside."""
    g, u = H[:, :I], H[:, I:]
    keep_g = keep_u = 1.0
    if limit > 0:
        keep_g = (g <= limit).astype(F64)
        keep_u = (np.abs(u) <= limit).astype(F64)
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    s = sigmoid(g)
    dg = dA * u * s * (1.0 + g * (1.0 - s)) * keep_g
    du = dA * g * s * keep_u
    return np.concatenate([dg, du], axis=1)


# --------------------------------------------------------------------------
# Layer forward: route -> dispatch -> expert MLPs -> combine
# --------------------------------------------------------------------------

def dispatch(x: np.ndarray, rt: dict) -> np.ndarray:
    """Xp[r] = x[token of row r]  (token sorting into expert order)."""
    return np.array(x, dtype=F64)[rt["src_of"] // rt["k"]]


def combine(rows: np.ndarray, rt: dict) -> np.ndarray:
    """out[t] = sum_j w_tj * rows[row_of[t*k + j]], slots in order."""
    T = rt["ids"].shape[0]
    k = rt["k"]
    out = np.zeros((T, rows.shape[1]), dtype=F64)
    for j in range(k):
        r = rt["row_of"][np.arange(T) * k + j]
        out += rt["w"][:, j:j + 1] * rows[r]
    return out


def forward(x, rt: dict, w_gate_up, w_down, expert_fn=None, limit: float = 0.0) -> dict:
    """Layer forward.  expert_fn(e, Xp_e) -> Y_e replaces the expert MLP when
    given (used by the identity-expert invariant)."""
    off = rt["offsets"]
    E = rt["E"]
    Xp = dispatch(x, rt)
    R = Xp.shape[0]
    if expert_fn is not None:
        Y = np.zeros((R, Xp.shape[1]), dtype=F64)
        for e in range(E):
            s = slice(off[e], off[e + 1])
            Y[s] = expert_fn(e, Xp[s])
        return dict(out=combine(Y, rt), Y=Y, Xp=Xp)
    Wgu = w_gate_up
    Wd = w_down
    I = Wgu.shape[1] // 2
    d = Wd.shape[1]
    H = np.zeros((R, 2 * I), dtype=F64)
    A = np.zeros((R, I), dtype=F64)
    Y = np.zeros((R, d), dtype=F64)
    for e in range(E):
        s = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        H[s] = Xp[s] @ np.asarray(Wgu[e], F64).T          # gate/up GEMM
        A[s] = swiglu(H[s], I, limit)                       # SwiGLU
        Y[s] = A[s] @ np.asarray(Wd[e], F64).T              # down GEMM
    return dict(out=combine(Y, rt), H=H, A=A, Y=Y, Xp=Xp)


# --------------------------------------------------------------------------
# Layer backward  [P1; P2 "Where MoE training loses time"]
# --------------------------------------------------------------------------

def backward(dout, rt: dict, w_gate_up, w_down, fwd: dict,
             logits=None, limit: float = 0.0) -> dict:
    """Exact gradient of L = sum(dout * out)."""
    dout = np.asarray(dout, F64)
    T, k, E = rt["ids"].shape[0], rt["k"], rt["E"]
    off, src_of, row_of = rt["offsets"], rt["src_of"], rt["row_of"]
    Wgu, Wd = w_gate_up, w_down
    I = Wgu.shape[1] // 2
    d = Wd.shape[1]
    R = src_of.size
    tok = src_of // k
    w_row = rt["w"].ravel()[src_of]                    # weight of each row

    # combine backward: gradient of each expert output row and of each weight
    dY = w_row[:, None] * dout[tok]
    Y = fwd["Y"]
    d_topk_w = np.einsum("td,tjd->tj", dout,
                         Y[row_of.reshape(T, k)])

    H, A, Xp = fwd["H"], fwd["A"], fwd["Xp"]
    dW_down = np.zeros((E, d, I), dtype=F64)
    dW_gate_up = np.zeros((E, 2 * I, d), dtype=F64)
    dXp = np.zeros((R, d), dtype=F64)
    for e in range(E):
        s = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue                                    # empty expert: dW = 0
        Wd_e = np.asarray(Wd[e], F64)
        Wgu_e = np.asarray(Wgu[e], F64)
        dA = dY[s] @ Wd_e                               # down dgrad
        dW_down[e] = dY[s].T @ A[s]                     # down wgrad
        dH = swiglu_backward(H[s], dA, I, limit)        # SwiGLU backward
        dXp[s] = dH @ Wgu_e                             # gate/up dgrad
        dW_gate_up[e] = dH.T @ Xp[s]                    # gate/up wgrad

    # dispatch backward: each token gathers its k rows' gradients
    dx = np.zeros((T, d), dtype=F64)
    for j in range(k):
        dx += dXp[row_of[np.arange(T) * k + j]]

    res = dict(dx=dx, dW_gate_up=dW_gate_up, dW_down=dW_down,
               d_topk_w=d_topk_w)
    if logits is not None:
        res["dlogits"] = router_logit_grad(rt, d_topk_w, logits.shape[1])
    return res


def router_logit_grad(rt: dict, d_topk_w: np.ndarray, E: int) -> np.ndarray:
    """Through w = softmax over the selected logits:
    dl_i = w_i (dw_i - sum_j w_j dw_j) for selected i, 0 for the rest."""
    w = rt["w"]
    inner = np.sum(w * d_topk_w, axis=1, keepdims=True)
    g_sel = w * (d_topk_w - inner)
    T = w.shape[0]
    dl = np.zeros((T, E), dtype=F64)
    np.put_along_axis(dl, rt["ids"], g_sel, axis=1)
    return dl


# --------------------------------------------------------------------------
# Per-token and per-expert evaluation (for sampled checks at full size).
# Same definitions as above, restricted to a subset.
# --------------------------------------------------------------------------

def forward_backward_tokens(x, logits, dout, w_gate_up, w_down, k: int,
                            tokens: np.ndarray, ids=None, w=None, limit: float = 0.0) -> dict:
    """out, dx, d_topk_w (and dlogits when logits are given) for a subset of
    tokens.  Every token's result depends only on its own routing and on the
    weights, so this evaluates the same definitions row by row."""
    tokens = np.asarray(tokens)
    E = w_gate_up.shape[0]
    I = w_gate_up.shape[1] // 2
    if logits is not None:
        lg = np.asarray(logits)[tokens]
        ids_t = topk_select(lg, k)
        w_t = topk_weights(lg, ids_t)
    else:
        ids_t = np.asarray(ids)[tokens].astype(np.int64)
        w_t = np.asarray(w, F64)[tokens]
    x_t = np.asarray(x, F64)[tokens]
    g_t = np.asarray(dout, F64)[tokens]
    n = tokens.size
    out = np.zeros_like(x_t)
    dx = np.zeros_like(x_t)
    dtw = np.zeros((n, k), dtype=F64)
    for i in range(n):
        for j in range(k):
            e = ids_t[i, j]
            Wgu_e = np.asarray(w_gate_up[e], F64)
            Wd_e = np.asarray(w_down[e], F64)
            h = Wgu_e @ x_t[i]
            a = swiglu(h[None, :], I, limit)[0]
            y = Wd_e @ a
            out[i] += w_t[i, j] * y
            dtw[i, j] = g_t[i] @ y
            dA = w_t[i, j] * (Wd_e.T @ g_t[i])
            dh = swiglu_backward(h[None, :], dA[None, :], I, limit)[0]
            dx[i] += Wgu_e.T @ dh
    res = dict(out=out, dx=dx, d_topk_w=dtw, ids=ids_t, w=w_t)
    if logits is not None:
        rt = dict(ids=ids_t, w=w_t)
        res["dlogits"] = router_logit_grad(rt, dtw, E)
    return res


def expert_weight_grads(x, dout, rt: dict, w_gate_up, w_down, e: int, limit: float = 0.0):
    """dW_gate_up[e], dW_down[e] from the rows routed to expert e."""
    k = rt["k"]
    s = slice(rt["offsets"][e], rt["offsets"][e + 1])
    src = rt["src_of"][s]
    Wgu_e = np.asarray(w_gate_up[e], F64)
    Wd_e = np.asarray(w_down[e], F64)
    I = Wgu_e.shape[0] // 2
    Xp = np.asarray(x, F64)[src // k]
    wr = rt["w"].ravel()[src]
    dY = wr[:, None] * np.asarray(dout, F64)[src // k]
    H = Xp @ Wgu_e.T
    A = swiglu(H, I, limit)
    dA = dY @ Wd_e
    dH = swiglu_backward(H, dA, I, limit)
    return dH.T @ Xp, dY.T @ A


# --------------------------------------------------------------------------
# Blockwise FP8 (OCP e4m3)  [P2 "Precision and hardware support"]
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3 value (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits, no infinities, largest finite 448), ties to even mantissa,
    saturating at +-448.  Input and output are float arrays holding the value,
    not the 8-bit code."""
    v = np.asarray(v, dtype=F64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    out = np.zeros_like(a)
    sub = a < 2.0 ** -6                       # subnormals: quantum 2^-9
    out[sub] = np.rint(a[sub] / 2.0 ** -9) * 2.0 ** -9
    nrm = ~sub
    _, ex = np.frexp(a[nrm])                  # a = m * 2^ex, m in [0.5, 1)
    quantum = np.ldexp(1.0, ex - 1 - 3)       # 3 mantissa bits below the leading 1
    out[nrm] = np.rint(a[nrm] / quantum) * quantum
    out = np.minimum(out, E4M3_MAX)
    return np.copysign(out, v)


def _quant_block(blk: np.ndarray) -> np.ndarray:
    """Quantise one block (any shape) with one scale; returns q*s as float64."""
    b32 = np.asarray(blk, dtype=np.float32)
    amax = np.float32(np.max(np.abs(b32))) if b32.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    q = e4m3_round(np.asarray(b32 / s, dtype=np.float32))
    return q * F64(s)


def quant_rows_1x128(X: np.ndarray) -> np.ndarray:
    """Activation blocks: 1 row x 128 consecutive columns (the K dimension)."""
    X = np.asarray(X)
    out = np.zeros(X.shape, dtype=F64)
    for c0 in range(0, X.shape[1], 128):
        blk = np.asarray(X[:, c0:c0 + 128], dtype=np.float32)
        amax = np.max(np.abs(blk), axis=1, keepdims=True).astype(np.float32)
        s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32),
                     np.float32(1.0)).astype(np.float32)
        q = e4m3_round((blk / s).astype(np.float32))
        out[:, c0:c0 + 128] = q * s.astype(F64)
    return out


def quant_weight_128x128(W: np.ndarray) -> np.ndarray:
    """Weight blocks: 128 x 128 tiles of one expert's [N, K] matrix."""
    W = np.asarray(W)
    out = np.zeros(W.shape, dtype=F64)
    for r0 in range(0, W.shape[0], 128):
        for c0 in range(0, W.shape[1], 128):
            out[r0:r0 + 128, c0:c0 + 128] = _quant_block(W[r0:r0 + 128, c0:c0 + 128])
    return out


def quant_tokens_128(X: np.ndarray) -> np.ndarray:
    """Weight-gradient operand blocks: 128 consecutive rows (tokens) x 1
    column, counted from the expert's first row; the last block may be short."""
    X = np.asarray(X)
    out = np.zeros(X.shape, dtype=F64)
    for r0 in range(0, X.shape[0], 128):
        out[r0:r0 + 128] = _quant_cols(X[r0:r0 + 128])
    return out


def _quant_cols(blk: np.ndarray) -> np.ndarray:
    b32 = np.asarray(blk, dtype=np.float32)
    amax = np.max(np.abs(b32), axis=0, keepdims=True).astype(np.float32)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    q = e4m3_round((b32 / s).astype(np.float32))
    return q * s.astype(F64)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), via the
    float32 value's bit pattern."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


# --------------------------------------------------------------------------
# MXFP8: OCP microscaling blocks of 32 values with a power-of-two (E8M0)
# scale and e4m3 elements  [P2 "Precision and hardware support": MXFP8 uses
# smaller scaling groups than blockwise FP8; P4 overview: the mxfp8 option]
# --------------------------------------------------------------------------

MX_BLOCK = 32
E4M3_EMAX = 8          # exponent of e4m3's largest binade: 448 = 1.75 * 2^8
E8M0_MIN = -127        # smallest exponent an E8M0 scale encodes


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent X of a block whose largest magnitude is amax (float32
    values): the smallest integer with amax <= 448 * 2^X, i.e. the blockwise
    scale amax / 448 rounded up to a power of two, so that no value of the
    block saturates; X >= -127 (the smallest E8M0 scale) and X = 0 for an
    all-zero block.  With amax = m * 2^e, m in [1, 2): X = e - 8, plus one
    when m > 1.75."""
    a = np.asarray(amax, dtype=np.float32).astype(F64)
    f, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    m, e = 2.0 * f, ex - 1
    X = np.maximum(e - E4M3_EMAX + (m > 1.75), E8M0_MIN)
    return np.where(a > 0, X, 0).astype(np.int64)


def mx_quant_last(X: np.ndarray):
    """1 x 32 blocks along the last axis (a multiple of 32 long).  Returns
    (element values q, exponents [.., n/32]); the block's values are
    q * 2^X with q the e4m3 value nearest to v / 2^X (ties to even)."""
    b = np.asarray(X, dtype=np.float32).astype(F64)
    sh = b.shape
    blk = b.reshape(sh[:-1] + (sh[-1] // MX_BLOCK, MX_BLOCK))
    ex = mx_scale_exponent(np.max(np.abs(blk), axis=-1))
    q = e4m3_round(np.ldexp(blk, -ex[..., None]))
    return q.reshape(sh), ex


def mx_rows(X: np.ndarray) -> np.ndarray:
    """Dequantised 1 x 32 blocks along rows (the K dimension of an
    activation, a gradient, or a weight in the forward GEMMs)."""
    q, ex = mx_quant_last(X)
    return np.ldexp(q, np.repeat(ex, MX_BLOCK, axis=-1))


def mx_cols(X: np.ndarray) -> np.ndarray:
    """Dequantised 32 x 1 blocks down the columns: a weight in the data-
    gradient GEMMs, whose contraction runs over the weight's rows."""
    return mx_rows(np.asarray(X).T).T


def mx_tokens(X: np.ndarray) -> np.ndarray:
    """Weight-gradient operand blocks: 32 consecutive rows (tokens) x 1
    column, counted from the expert's first row; the last block may be short
    (zero padding leaves its largest magnitude unchanged)."""
    X = np.asarray(X)
    n = X.shape[0]
    pad = np.zeros((-(-n // MX_BLOCK) * MX_BLOCK,) + X.shape[1:], dtype=np.float32)
    pad[:n] = X
    return mx_cols(pad)[:n]


# Quantisation recipes of the fp8 layers: which block shape each GEMM operand
# takes.  act: activations and gradients, blocks along their K (last) axis;
# w_fwd: a weight [N, K] in the forward GEMMs (contraction over K); w_bwd: the
# same weight in a data-gradient GEMM (contraction over N); tok: both operands
# of a weight gradient (contraction over the expert's tokens).
FP8_BLOCK = dict(act=quant_rows_1x128, w_fwd=quant_weight_128x128,
                 w_bwd=quant_weight_128x128, tok=quant_tokens_128)
MXFP8 = dict(act=mx_rows, w_fwd=mx_rows, w_bwd=mx_cols, tok=mx_tokens)


def no_quant(X: np.ndarray) -> np.ndarray:
    """The identity encoding: operands enter the GEMM unquantised."""
    return np.asarray(X, dtype=F64)


# Unquantised GEMM operands: forward_fp8 with this recipe is the forward of
# the bf16 layer (H and Aw stored in bf16), the forward half of fp8_bwd.
NO_QUANT = dict(act=no_quant, w_fwd=no_quant, w_bwd=no_quant, tok=no_quant)


def forward_fp8(x, rt: dict, w_gate_up, w_down, recipe=FP8_BLOCK, limit: float = 0.0) -> dict:
    """Forward with both GEMMs on block-quantised e4m3 operands (block
    shapes from `recipe`: FP8_BLOCK or MXFP8).  The top-k
    weight of each row is folded into the SwiGLU output before the down GEMM
    (Aw = w * silu(g) * up, stored bf16), so the combine is a plain sum."""
    off, E = rt["offsets"], rt["E"]
    Xp = dispatch(x, rt)
    R = Xp.shape[0]
    I = w_gate_up.shape[1] // 2
    d = w_down.shape[1]
    w_row = rt["w"].ravel()[rt["src_of"]]
    H = np.zeros((R, 2 * I))
    Aw = np.zeros((R, I))
    Yw = np.zeros((R, d))
    for e in range(E):
        s = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        Hs = recipe["act"](Xp[s]) @ recipe["w_fwd"](w_gate_up[e]).T
        Aw[s] = bf16_round(w_row[s, None] * swiglu(Hs, I, limit))
        H[s] = bf16_round(Hs)
        Yw[s] = recipe["act"](Aw[s]) @ recipe["w_fwd"](w_down[e]).T
    T, k = rt["ids"].shape
    out = np.zeros((T, d))
    for j in range(k):
        out += Yw[rt["row_of"][np.arange(T) * k + j]]
    return dict(out=out, H=H, Aw=Aw, Yw=Yw, Xp=Xp)


def backward_fp8(dout, rt: dict, w_gate_up, w_down, fwd: dict,
                 logits=None, recipe=FP8_BLOCK, limit: float = 0.0) -> dict:
    """Backward with all four GEMMs on block-quantised e4m3 operands.  The
    top-k-weight gradient is <G_r, a_r> with G_r the quantised down dgrad
    (the backward's estimate of W_down^T dout_t) and a_r = silu(g) * up from
    the stored H; the down wgrad quantises dout and Aw in token blocks."""
    dout = np.asarray(dout, F64)
    T, k, E = rt["ids"].shape[0], rt["k"], rt["E"]
    off, src_of, row_of = rt["offsets"], rt["src_of"], rt["row_of"]
    I = w_gate_up.shape[1] // 2
    d = w_down.shape[1]
    R = src_of.size
    tok = src_of // k
    w_row = rt["w"].ravel()[src_of]
    H, Aw, Xp = fwd["H"], fwd["Aw"], fwd["Xp"]
    dw_row = np.zeros(R)
    dW_down = np.zeros((E, d, I))
    dW_gate_up = np.zeros((E, 2 * I, d))
    dXp = np.zeros((R, d))
    for e in range(E):
        s = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        Wd_q = recipe["w_bwd"](w_down[e])
        Wgu_q = recipe["w_bwd"](w_gate_up[e])
        G = recipe["act"](dout[tok[s]]) @ Wd_q               # down dgrad
        dw_row[s] = np.sum(G * swiglu(H[s], I, limit), axis=1)
        dA = w_row[s, None] * G
        dW_down[e] = recipe["tok"](dout[tok[s]]).T @ recipe["tok"](Aw[s])
        dH = bf16_round(swiglu_backward(H[s], dA, I, limit))
        dXp[s] = recipe["act"](dH) @ Wgu_q                    # gate/up dgrad
        dW_gate_up[e] = recipe["tok"](dH).T @ recipe["tok"](Xp[s])
    d_topk_w = dw_row[row_of].reshape(T, k)
    dx = np.zeros((T, d))
    for j in range(k):
        dx += dXp[row_of[np.arange(T) * k + j]]
    res = dict(dx=dx, dW_gate_up=dW_gate_up, dW_down=dW_down, d_topk_w=d_topk_w)
    if logits is not None:
        res["dlogits"] = router_logit_grad(rt, d_topk_w, logits.shape[1])
    return res


def encode_expert_weights(w_gate_up, w_down, e: int, recipe=FP8_BLOCK, fwd_recipe=None):
    """Expert e's weights as the fp8 layer's GEMMs see them: (gate/up, down)
    in the forward encoding of fwd_recipe (default recipe), then in the
    data-gradient encoding of recipe."""
    fr = recipe if fwd_recipe is None else fwd_recipe
    fw = (fr["w_fwd"](w_gate_up[e]), fr["w_fwd"](w_down[e]))
    bw = fw if recipe["w_bwd"] is fr["w_fwd"] else \
        (recipe["w_bwd"](w_gate_up[e]), recipe["w_bwd"](w_down[e]))
    return fw + bw


def forward_backward_tokens_fp8(x, logits, dout, w_gate_up, w_down, k: int,
                                tokens: np.ndarray, ids=None, w=None,
                                recipe=FP8_BLOCK, fwd_recipe=None, encoded=None,
                                limit: float = 0.0) -> dict:
    """forward_fp8 (with fwd_recipe, default recipe) / backward_fp8 (with
    recipe) results (out, dx, d_topk_w, dlogits) for a subset of tokens.  Activation blocks lie within one row and weight
    blocks depend only on the weights, so each token's results follow from
    its own rows; the same steps as the full functions, row by row.
    encoded: optional {expert: encode_expert_weights(...)} computed ahead
    (for instance in parallel) with the same recipes."""
    tokens = np.asarray(tokens)
    E = w_gate_up.shape[0]
    I = w_gate_up.shape[1] // 2
    if logits is not None:
        lg = np.asarray(logits)[tokens]
        ids_t = topk_select(lg, k)
        w_t = topk_weights(lg, ids_t)
    else:
        ids_t = np.asarray(ids)[tokens].astype(np.int64)
        w_t = np.asarray(w, F64)[tokens]
    fr = recipe if fwd_recipe is None else fwd_recipe
    qw = dict(encoded) if encoded is not None else {}

    def weights(e):  # (gate/up, down) forward and data-gradient forms
        if e not in qw:
            qw[e] = encode_expert_weights(w_gate_up, w_down, e, recipe, fwd_recipe)
        return qw[e]

    n, d = tokens.size, w_down.shape[1]
    out, dx = np.zeros((n, d)), np.zeros((n, d))
    dtw = np.zeros((n, k))
    for i, t in enumerate(tokens):
        xq = fr["act"](np.asarray(x, F64)[t][None, :])
        gq = recipe["act"](np.asarray(dout, F64)[t][None, :])
        for j in range(k):
            Wgu_f, Wd_f, Wgu_b, Wd_b = weights(ids_t[i, j])
            Hs = xq @ Wgu_f.T
            H = bf16_round(Hs)
            Aw = bf16_round(w_t[i, j] * swiglu(Hs, I, limit))
            out[i] += (fr["act"](Aw) @ Wd_f.T)[0]
            G = gq @ Wd_b
            dtw[i, j] = np.sum(G * swiglu(H, I, limit))
            dH = bf16_round(swiglu_backward(H, w_t[i, j] * G, I, limit))
            dx[i] += (recipe["act"](dH) @ Wgu_b)[0]
    res = dict(out=out, dx=dx, d_topk_w=dtw, ids=ids_t, w=w_t)
    if logits is not None:
        res["dlogits"] = router_logit_grad(dict(ids=ids_t, w=w_t), dtw, E)
    return res


def expert_weight_grads_fp8(x, dout, rt: dict, w_gate_up, w_down, e: int,
                            recipe=FP8_BLOCK, fwd_recipe=None, limit: float = 0.0):
    """backward_fp8's dW_gate_up[e], dW_down[e] from the rows of expert e
    alone (token blocks are counted from the expert's first row); the
    forward's H and Aw with fwd_recipe (default recipe)."""
    fr = recipe if fwd_recipe is None else fwd_recipe
    k = rt["k"]
    s = slice(rt["offsets"][e], rt["offsets"][e + 1])
    src = rt["src_of"][s]
    I = w_gate_up.shape[1] // 2
    Wgu_f = fr["w_fwd"](w_gate_up[e])
    Wd_b = recipe["w_bwd"](w_down[e])
    Xp = np.asarray(x, F64)[src // k]
    g = np.asarray(dout, F64)[src // k]
    wr = rt["w"].ravel()[src]
    Hs = fr["act"](Xp) @ Wgu_f.T
    H = bf16_round(Hs)
    Aw = bf16_round(wr[:, None] * swiglu(Hs, I, limit))
    G = recipe["act"](g) @ Wd_b
    dH = bf16_round(swiglu_backward(H, wr[:, None] * G, I, limit))
    dW_down = recipe["tok"](g).T @ recipe["tok"](Aw)
    dW_gate_up = recipe["tok"](dH).T @ recipe["tok"](Xp)
    return dW_gate_up, dW_down
