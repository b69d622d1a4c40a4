"""The fused MoE layer as PyTorch operators with autograd.

The pages' integration registers the layer's backward as a custom operator
so that the compiler accepts the tensors the forward saves, and runs the
layer under activation checkpointing ("Mario/overlap moe kernel
integration", overview and commits on the custom autograd ops;
"Prime Intellect added the missing backward pass to DeepSeek's fused MoE
kernel ...").  Here:

* ``ctr_moe::moe_fwd`` and ``ctr_moe::moe_bwd`` are ``torch.library`` custom
  operators over ``moe_forward`` / ``moe_backward`` of the C ABI, with fake
  (shape-only) implementations, so ``torch.compile(fullgraph=True)`` traces
  through them without graph breaks;
* ``moe_fwd`` carries an autograd formula that calls ``moe_bwd``;
* ``recompute=True`` keeps nothing from the forward: the backward reruns the
  gate/up GEMM from x (``moe_backward`` with ``saved == NULL``).

Every call allocates its outputs and workspace from torch's caching
allocator on the inputs' device and enqueues on torch's current stream.
Routing comes from router logits; the gradient reaches them through the
renormalised top-k softmax.
"""
from __future__ import annotations

import ctypes

import torch
from torch import Tensor

from . import binding as B

_NS = "ctr_moe"


_FLOATS = (torch.float32, torch.bfloat16)


def _require(ok: bool, msg: str):
    if not ok:
        raise ValueError(msg)


def _check_layer_args(x: Tensor, logits: Tensor, w_gate_up: Tensor, w_down: Tensor, k: int,
                      precision: str):
    """Shapes, dtypes and contiguity of the layer's inputs, checked before
    anything is launched: x [T,d], logits [T,E], w_gate_up [E,2I,d],
    w_down [E,d,I], 1 <= k <= E."""
    _require(x.dim() == 2, f"x must be [T, d], got {tuple(x.shape)}")
    T, d = x.shape
    _require(w_gate_up.dim() == 3 and w_gate_up.shape[2] == d and w_gate_up.shape[1] % 2 == 0,
             f"w_gate_up must be [E, 2I, d={d}], got {tuple(w_gate_up.shape)}")
    E, two_i, _ = w_gate_up.shape
    _require(tuple(w_down.shape) == (E, d, two_i // 2),
             f"w_down must be [E={E}, d={d}, I={two_i // 2}], got {tuple(w_down.shape)}")
    _require(tuple(logits.shape) == (T, E), f"logits must be [T={T}, E={E}], got {tuple(logits.shape)}")
    _require(1 <= k <= E, f"k={k} outside [1, E={E}]")
    _require(precision in B._PREC, f"precision {precision!r} unknown")
    _require(x.dtype in _FLOATS and w_gate_up.dtype == x.dtype and w_down.dtype == x.dtype,
             f"x and both weights need one dtype of {_FLOATS}, got {x.dtype}, {w_gate_up.dtype}, "
             f"{w_down.dtype}")
    _require(logits.dtype in _FLOATS, f"logits dtype {logits.dtype} not in {_FLOATS}")
    for name, t in (("x", x), ("logits", logits), ("w_gate_up", w_gate_up), ("w_down", w_down)):
        _require(t.is_contiguous(), f"{name} must be contiguous")


def _check_devices(**tensors):
    """Every tensor on the first one's GPU (checked last, after the shapes)."""
    dev = next(iter(tensors.values())).device
    for name, t in tensors.items():
        _require(t.device.type == "cuda" and t.device == dev, f"{name} is on {t.device}; every tensor "
                 f"must be on one GPU ({dev})")


def _check_backward_args(dout: Tensor, x: Tensor, saved: Tensor, routing, k: int, precision: str):
    """dout [T,d] in x's dtype, `saved` empty or of the forward's size, and the
    routing tensors the forward returned, on x's device."""
    T, d = x.shape
    _require(tuple(dout.shape) == (T, d) and dout.dtype == x.dtype,
             f"dout must be [T={T}, d={d}] {x.dtype}, got {tuple(dout.shape)} {dout.dtype}")
    ids, w, counts, offsets, row_of, src_of = routing
    E = counts.numel()
    for name, t, shape, dt in (("topk_ids", ids, (T, k), torch.int32), ("topk_w", w, (T, k), torch.float32),
                               ("counts", counts, (E,), torch.int32), ("offsets", offsets, (E + 1,), torch.int32),
                               ("row_of", row_of, (T * k,), torch.int32), ("src_of", src_of, (T * k,), torch.int32),
                               ("saved", saved, (saved.numel(),), torch.uint8)):
        _require(tuple(t.shape) == shape and t.dtype == dt, f"{name} must be {shape} {dt}, got "
                 f"{tuple(t.shape)} {t.dtype}")
        _require(t.is_contiguous(), f"{name} must be contiguous")


def _shape(x: Tensor, logits: Tensor, w_gate_up: Tensor, k: int, precision: str, swiglu_limit: float = 0.0):
    T, d = x.shape
    E, two_i, _ = w_gate_up.shape
    return B.make_shape(T, d, E, k, two_i // 2, x.dtype, logits.dtype, precision, swiglu_limit)


def _workspace(shape, op, device) -> Tensor:
    return torch.empty(B.workspace_size(shape, op), dtype=torch.uint8, device=device)


def _routing_empty(T, E, k, device):
    i32 = dict(dtype=torch.int32, device=device)
    return (torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
            torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32),
            torch.empty(T * k, **i32))


@torch.library.custom_op(f"{_NS}::moe_fwd", mutates_args=())
def moe_fwd(x: Tensor, logits: Tensor, w_gate_up: Tensor, w_down: Tensor, k: int, precision: str,
            save: bool, swiglu_limit: float = 0.0
            ) -> tuple[Tensor, Tensor, Tensor, Tensor, Tensor, Tensor, Tensor, Tensor]:
    """Layer forward.  Returns (out [T,d], saved (uint8; empty unless save),
    topk_ids, topk_w, counts, offsets, row_of, src_of).  swiglu_limit > 0:
    the clamped SwiGLU."""
    _check_layer_args(x, logits, w_gate_up, w_down, k, precision)
    _check_devices(x=x, logits=logits, w_gate_up=w_gate_up, w_down=w_down)
    shape = _shape(x, logits, w_gate_up, k, precision, swiglu_limit)
    T, d = x.shape
    E = w_gate_up.shape[0]
    dev = x.device
    out = torch.empty((T, d), dtype=x.dtype, device=dev)
    saved = torch.empty(B.saved_size(shape) if save else 0, dtype=torch.uint8, device=dev)
    rt = _routing_empty(T, E, k, dev)
    r = B.Routing(*rt, logits=logits)
    cr = r.c()
    ws = _workspace(shape, B.OP_FORWARD, dev)
    B._check("moe_forward", B.lib().moe_forward(
        ctypes.byref(shape), B._ptr(x), ctypes.byref(cr), B._ptr(w_gate_up), B._ptr(w_down), B._ptr(out),
        B._ptr(saved) if save else None, B._ptr(ws), ws.numel(), B._stream(dev)))
    return (out, saved) + rt


@moe_fwd.register_fake
def _(x, logits, w_gate_up, w_down, k, precision, save, swiglu_limit=0.0):
    T, d = x.shape
    E = w_gate_up.shape[0]
    shape = _shape(x, logits, w_gate_up, k, precision, swiglu_limit)
    n = B.saved_size(shape) if save else 0
    i32 = dict(dtype=torch.int32)
    return (x.new_empty((T, d)), x.new_empty((n,), dtype=torch.uint8), x.new_empty((T, k), **i32),
            x.new_empty((T, k), dtype=torch.float32), x.new_empty((E,), **i32),
            x.new_empty((E + 1,), **i32), x.new_empty((T * k,), **i32), x.new_empty((T * k,), **i32))


@torch.library.custom_op(f"{_NS}::moe_bwd", mutates_args=())
def moe_bwd(dout: Tensor, x: Tensor, logits: Tensor, w_gate_up: Tensor, w_down: Tensor, saved: Tensor,
            topk_ids: Tensor, topk_w: Tensor, counts: Tensor, offsets: Tensor, row_of: Tensor,
            src_of: Tensor, k: int, precision: str, swiglu_limit: float = 0.0
            ) -> tuple[Tensor, Tensor, Tensor, Tensor]:
    """Layer backward: (dx, dlogits, dw_gate_up, dw_down).  An empty `saved`
    selects recomputation."""
    _check_layer_args(x, logits, w_gate_up, w_down, k, precision)
    dout = dout.contiguous()
    _check_backward_args(dout, x, saved, (topk_ids, topk_w, counts, offsets, row_of, src_of), k, precision)
    shape = _shape(x, logits, w_gate_up, k, precision, swiglu_limit)
    _require(saved.numel() in (0, B.saved_size(shape)),
             f"saved holds {saved.numel()} bytes, expected 0 or {B.saved_size(shape)}")
    _check_devices(x=x, dout=dout, logits=logits, w_gate_up=w_gate_up, w_down=w_down, saved=saved,
                   topk_ids=topk_ids, topk_w=topk_w, counts=counts, offsets=offsets, row_of=row_of,
                   src_of=src_of)
    T, d = x.shape
    E, two_i, _ = w_gate_up.shape
    dev = x.device
    recompute = saved.numel() == 0
    dx = torch.empty_like(x)
    dlogits = torch.empty_like(logits)
    dwgu = torch.empty_like(w_gate_up)
    dwd = torch.empty_like(w_down)
    d_topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    r = B.Routing(topk_ids, topk_w, counts, offsets, row_of, src_of, logits=logits)
    cr = r.c()
    ws = _workspace(shape, B.OP_BACKWARD_RECOMPUTE if recompute else B.OP_BACKWARD, dev)
    B._check("moe_backward", B.lib().moe_backward(
        ctypes.byref(shape), B._ptr(dout), B._ptr(x), ctypes.byref(cr), B._ptr(w_gate_up), B._ptr(w_down),
        None if recompute else B._ptr(saved), B._ptr(dx), B._ptr(dwgu), B._ptr(dwd), B._ptr(d_topk_w),
        B._ptr(dlogits), B._ptr(ws), ws.numel(), B._stream(dev)))
    return dx, dlogits, dwgu, dwd


@moe_bwd.register_fake
def _(dout, x, logits, w_gate_up, w_down, saved, topk_ids, topk_w, counts, offsets, row_of, src_of,
      k, precision, swiglu_limit=0.0):
    return (torch.empty_like(x), torch.empty_like(logits), torch.empty_like(w_gate_up),
            torch.empty_like(w_down))


def _setup_context(ctx, inputs, output):
    x, logits, w_gate_up, w_down, k, precision, save, swiglu_limit = inputs
    ctx.save_for_backward(x, logits, w_gate_up, w_down, *output[1:])
    ctx.k, ctx.precision, ctx.swiglu_limit = k, precision, swiglu_limit


def _backward(ctx, dout, *unused):
    x, logits, w_gate_up, w_down, saved, ids, w, counts, offsets, row_of, src_of = ctx.saved_tensors
    dx, dlogits, dwgu, dwd = moe_bwd(dout, x, logits, w_gate_up, w_down, saved, ids, w, counts, offsets,
                                     row_of, src_of, ctx.k, ctx.precision, ctx.swiglu_limit)
    return dx, dlogits, dwgu, dwd, None, None, None, None


moe_fwd.register_autograd(_backward, setup_context=_setup_context)


def moe_layer(x: Tensor, logits: Tensor, w_gate_up: Tensor, w_down: Tensor, k: int,
              precision: str = "native", recompute: bool = False, swiglu_limit: float = 0.0) -> Tensor:
    """out [T,d] of the layer, differentiable in x, logits and both weights.
    recompute=True: activation checkpointing inside the operator (nothing
    kept between forward and backward but the routing).  swiglu_limit > 0:
    the clamped SwiGLU with that limit."""
    for name, t in (("x", x), ("logits", logits), ("w_gate_up", w_gate_up), ("w_down", w_down)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return moe_fwd(x, logits, w_gate_up, w_down, k, precision, not recompute, swiglu_limit)[0]
