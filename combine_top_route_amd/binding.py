"""Python binding of the C ABI in include/moe.h (ctypes).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), their device pointers and torch's current HIP stream are handed
to the library, and a non-OK status raises.  Every step of the layer runs in
the library's HIP kernels; there is no fallback.  PyTorch supplies device
memory (outputs, workspace) and the stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
PREC_NATIVE, PREC_FP8_BLOCK, PREC_MXFP8, PREC_FP8_BWD = 0, 1, 2, 3
OP_ROUTE, OP_FORWARD, OP_BACKWARD, OP_BACKWARD_RECOMPUTE = 0, 1, 2, 3
QUANT_ROWS, QUANT_WEIGHT, QUANT_WEIGHT_T = 0, 1, 2

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_TORCH = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}
_PREC = {"native": PREC_NATIVE, "fp8_block": PREC_FP8_BLOCK, "mxfp8": PREC_MXFP8, "fp8_bwd": PREC_FP8_BWD}


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("I", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float), ("flags", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("row_of", ctypes.c_void_p),
                ("src_of", ctypes.c_void_p)]


class MoeKernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


# exported entry points: (name, restype, argtypes)
_P = ctypes.c_void_p
_SIGS = [
    ("moe_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(MoeShape), ctypes.c_int]),
    ("moe_saved_bytes", ctypes.c_size_t, [ctypes.POINTER(MoeShape)]),
    ("moe_workspace_size", ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    ("moe_saved_size", ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(ctypes.c_size_t)]),
    ("moe_route", ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeRouting), _P, ctypes.c_size_t, _P]),
    ("moe_route_noalloc", ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeRouting), _P]),
    ("moe_forward", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.POINTER(MoeRouting), _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]),
    ("moe_backward", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, ctypes.POINTER(MoeRouting), _P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("moe_permute", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.POINTER(MoeRouting), _P, _P]),
    ("moe_combine", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.POINTER(MoeRouting), _P, _P]),
    ("moe_quantize_fp8", ctypes.c_int, [ctypes.c_int, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                        _P]),
    ("moe_quantize_tokens_fp8", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_int64, ctypes.c_int,
                                               ctypes.POINTER(MoeRouting), _P, _P, _P, ctypes.c_size_t, _P]),
    ("moe_quantize_mxfp8", ctypes.c_int, [ctypes.c_int, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P,
                                          _P, _P]),
    ("moe_quantize_tokens_mxfp8", ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_int64, ctypes.c_int,
                                                 ctypes.POINTER(MoeRouting), _P, _P, _P, ctypes.c_size_t, _P]),
    ("moe_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("moe_last_error", ctypes.c_char_p, []),
    ("moe_profile_begin", ctypes.c_int, []),
    ("moe_profile_end", ctypes.c_int, [ctypes.POINTER(MoeKernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"MoE HIP library not built ({LIB_PATH} missing): "
                               "run `python -m combine_top_route_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        l = lib()
        self.status = status
        super().__init__(f"{call}: {l.moe_status_string(status).decode()}: "
                         f"{l.moe_last_error().decode()}")


def _check(call: str, status: int):
    if status != 0:
        raise MoeError(call, status)


FLAG_PERSISTENT = 1


def make_shape(T, d, E, k, I, dtype=torch.bfloat16, logits_dtype=None, precision="native",
               swiglu_limit=0.0, persistent=False) -> MoeShape:
    """swiglu_limit > 0: the clamped SwiGLU with that limit; persistent: the
    bf16 GEMMs as persistent kernels (MOE_FLAG_PERSISTENT; see moe.h)."""
    logits_dtype = dtype if logits_dtype is None else logits_dtype
    return MoeShape(T, d, E, k, I, _DT[dtype], _DT[logits_dtype], _PREC[precision], float(swiglu_limit),
                    FLAG_PERSISTENT if persistent else 0)


def workspace_size(shape: MoeShape, op: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(shape), op)
    if n == 0:
        raise ValueError(f"moe_workspace_bytes: {lib().moe_last_error().decode()}")
    return n


def saved_size(shape: MoeShape) -> int:
    n = lib().moe_saved_bytes(ctypes.byref(shape))
    if n == 0:
        raise ValueError(f"moe_saved_bytes: {lib().moe_last_error().decode()}")
    return n


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class Routing:
    """Routing tensors on the device (see moe_routing in include/moe.h)."""
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_of: torch.Tensor
    src_of: torch.Tensor
    logits: torch.Tensor | None = None

    @staticmethod
    def empty(T, E, k, device, logits=None, topk_ids=None, topk_w=None) -> "Routing":
        i32 = dict(dtype=torch.int32, device=device)
        return Routing(
            topk_ids=torch.empty((T, k), **i32) if topk_ids is None else topk_ids,
            topk_w=torch.empty((T, k), dtype=torch.float32, device=device) if topk_w is None else topk_w,
            counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
            row_of=torch.empty(T * k, **i32), src_of=torch.empty(T * k, **i32), logits=logits)

    def c(self) -> MoeRouting:
        return MoeRouting(_ptr(self.logits), _ptr(self.topk_ids), _ptr(self.topk_w), _ptr(self.counts),
                          _ptr(self.offsets), _ptr(self.row_of), _ptr(self.src_of))


class MoeLayer:
    """One layer shape with preallocated outputs and workspaces, so repeated
    calls (benchmarks, training loops) allocate nothing.  save=False: the
    forward keeps nothing and the backward recomputes H and Aw from x
    (activation checkpointing)."""

    def __init__(self, T, d, E, k, I, dtype=torch.bfloat16, logits_dtype=None,
                 precision="native", device="cuda", save=True, swiglu_limit=0.0, persistent=False):
        self.T, self.d, self.E, self.k, self.I = T, d, E, k, I
        self.dtype = dtype
        self.logits_dtype = dtype if logits_dtype is None else logits_dtype
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.shape = make_shape(T, d, E, k, I, dtype, self.logits_dtype, precision, swiglu_limit, persistent)
        dev = self.device
        self.ws_fwd = torch.empty(workspace_size(self.shape, OP_FORWARD), dtype=torch.uint8, device=dev)
        self.ws_bwd = torch.empty(workspace_size(self.shape, OP_BACKWARD if save else OP_BACKWARD_RECOMPUTE),
                                  dtype=torch.uint8, device=dev)
        self.saved = (torch.empty(saved_size(self.shape), dtype=torch.uint8, device=dev) if save else None)
        self.out = torch.empty((T, d), dtype=dtype, device=dev)
        self.routing = Routing.empty(T, E, k, dev)
        self.dx = torch.empty((T, d), dtype=dtype, device=dev)
        self.dw_gate_up = torch.empty((E, 2 * I, d), dtype=dtype, device=dev)
        self.dw_down = torch.empty((E, d, I), dtype=dtype, device=dev)
        self.d_topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.dlogits = torch.empty((T, E), dtype=self.logits_dtype, device=dev)

    def saved_views(self):
        """(H [R,2I], A [R,I]) views of the saved buffer."""
        R, I = self.T * self.k, self.I
        flat = self.saved.view(self.dtype)
        return flat[:R * 2 * I].view(R, 2 * I), flat[R * 2 * I:].view(R, I)

    def forward(self, x, w_gate_up, w_down, logits=None, topk_ids=None, topk_w=None):
        T, d, E, k, I, dt, dev = self.T, self.d, self.E, self.k, self.I, self.dtype, self.device
        _need(x, "x", (T, d), dt, dev)
        _need(w_gate_up, "w_gate_up", (E, 2 * I, d), dt, dev)
        _need(w_down, "w_down", (E, d, I), dt, dev)
        r = self.routing
        if logits is not None:
            _need(logits, "logits", (T, E), self.logits_dtype, dev)
            r.logits = logits
        else:
            _need(topk_ids, "topk_ids", (T, k), torch.int32, dev)
            _need(topk_w, "topk_w", (T, k), torch.float32, dev)
            r.logits = None
            r.topk_ids, r.topk_w = topk_ids, topk_w
        cr = r.c()
        _check("moe_forward", lib().moe_forward(
            ctypes.byref(self.shape), _ptr(x), ctypes.byref(cr), _ptr(w_gate_up), _ptr(w_down),
            _ptr(self.out), _ptr(self.saved), _ptr(self.ws_fwd), self.ws_fwd.numel(), _stream(dev)))
        return self.out

    def backward(self, dout, x, w_gate_up, w_down, want_dlogits=True):
        T, d, dt, dev = self.T, self.d, self.dtype, self.device
        _need(dout, "dout", (T, d), dt, dev)
        r = self.routing
        cr = r.c()
        dl = self.dlogits if (want_dlogits and r.logits is not None) else None
        _check("moe_backward", lib().moe_backward(
            ctypes.byref(self.shape), _ptr(dout), _ptr(x), ctypes.byref(cr), _ptr(w_gate_up),
            _ptr(w_down), _ptr(self.saved), _ptr(self.dx), _ptr(self.dw_gate_up), _ptr(self.dw_down),
            _ptr(self.d_topk_w), _ptr(dl), _ptr(self.ws_bwd), self.ws_bwd.numel(), _stream(dev)))
        res = dict(dx=self.dx, dW_gate_up=self.dw_gate_up, dW_down=self.dw_down, d_topk_w=self.d_topk_w)
        if dl is not None:
            res["dlogits"] = dl
        return res


def route(logits, k):
    """Routing alone from router logits [T,E] (f32 or bf16)."""
    T, E = logits.shape
    dev = logits.device
    shape = make_shape(T, 8, E, k, 8, torch.bfloat16, logits.dtype)
    r = Routing.empty(T, E, k, dev, logits=logits)
    ws = torch.empty(workspace_size(shape, OP_ROUTE), dtype=torch.uint8, device=dev)
    cr = r.c()
    _check("moe_route", lib().moe_route(ctypes.byref(shape), ctypes.byref(cr), _ptr(ws), ws.numel(),
                                         _stream(dev)))
    return r


def route_ids(topk_ids, topk_w, E):
    """Routing artefacts for given ids and weights (ids-in form)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _need(topk_w, "topk_w", (T, k), torch.float32, dev)
    shape = make_shape(T, 8, E, k, 8, torch.bfloat16)
    r = Routing.empty(T, E, k, dev, topk_ids=topk_ids, topk_w=topk_w)
    ws = torch.empty(workspace_size(shape, OP_ROUTE), dtype=torch.uint8, device=dev)
    cr = r.c()
    _check("moe_route", lib().moe_route(ctypes.byref(shape), ctypes.byref(cr), _ptr(ws), ws.numel(),
                                         _stream(dev)))
    return r


def route_noalloc(r: Routing, T, E, k, logits_dtype=torch.bfloat16):
    """moe_route_noalloc into the caller's routing tensors r (logits in when
    r.logits is set, else r.topk_ids / r.topk_w in); no workspace."""
    shape = make_shape(T, 8, E, k, 8, torch.bfloat16, logits_dtype)
    cr = r.c()
    _check("moe_route_noalloc", lib().moe_route_noalloc(ctypes.byref(shape), ctypes.byref(cr),
                                                         _stream(r.counts.device)))
    return r


def permute(x, routing: Routing, k, out=None):
    """Dispatch: xp [T*k, d] with xp[r] = x[src_of[r] / k] (into `out` when given)."""
    T, d = x.shape
    E = routing.counts.numel()
    shape = make_shape(T, d, E, k, 8, x.dtype)
    xp = torch.empty((T * k, d), dtype=x.dtype, device=x.device) if out is None else out
    _need(xp, "out", (T * k, d), x.dtype, x.device)
    cr = routing.c()
    _check("moe_permute", lib().moe_permute(ctypes.byref(shape), _ptr(x), ctypes.byref(cr), _ptr(xp),
                                             _stream(x.device)))
    return xp


def combine(rows, routing: Routing, T, k):
    d = rows.shape[1]
    E = routing.counts.numel()
    shape = make_shape(T, d, E, k, 8, rows.dtype)
    out = torch.empty((T, d), dtype=rows.dtype, device=rows.device)
    cr = routing.c()
    _check("moe_combine", lib().moe_combine(ctypes.byref(shape), _ptr(rows), ctypes.byref(cr), _ptr(out),
                                             _stream(rows.device)))
    return out


def profile_begin():
    _check("moe_profile_begin", lib().moe_profile_begin())


def profile_end() -> dict:
    """{kernel name: (launches, total ms)} of the launches since profile_begin."""
    cap = 64
    arr = (MoeKernelStat * cap)()
    n = ctypes.c_int()
    _check("moe_profile_end", lib().moe_profile_end(arr, cap, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n.value, cap))}


def quantize_fp8(src, kind=QUANT_ROWS):
    """e4m3 codes (uint8) and float32 scales of a bf16 tensor: kind
    QUANT_ROWS for [n0, n1] (1x128 blocks), QUANT_WEIGHT / QUANT_WEIGHT_T for
    [n0, n1, n2] (128x128 blocks, written as is or transposed)."""
    dev = src.device
    if src.dtype != torch.bfloat16 or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 tensor")
    if kind == QUANT_ROWS:
        n0, n1 = src.shape
        n2 = 0
        q = torch.empty((n0, n1), dtype=torch.uint8, device=dev)
        s = torch.empty((n0, n1 // 128), dtype=torch.float32, device=dev)
    else:
        n0, n1, n2 = src.shape
        qs = (n0, n1, n2) if kind == QUANT_WEIGHT else (n0, n2, n1)
        q = torch.empty(qs, dtype=torch.uint8, device=dev)
        s = torch.empty((qs[0], qs[1] // 128, qs[2] // 128), dtype=torch.float32, device=dev)
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(kind, _ptr(src), n0, n1, n2, _ptr(q), _ptr(s),
                                                      _stream(dev)))
    return q, s


def quantize_tokens_fp8(src, routing: Routing, T, k, gather):
    """Token-block codes q [C, 128 nblk] and scales s [C, nblk] of a
    weight-gradient operand (see moe_quantize_tokens_fp8); nblk =
    ceil(T*k/128) + E."""
    dev = src.device
    C = src.shape[1]
    E = routing.counts.numel()
    shape = make_shape(T, C, E, k, 128, torch.bfloat16)
    nblk = -(-T * k // 128) + E
    q = torch.zeros((C, 128 * nblk), dtype=torch.uint8, device=dev)
    s = torch.zeros((C, nblk), dtype=torch.float32, device=dev)
    ws = torch.empty(workspace_size(shape, OP_ROUTE), dtype=torch.uint8, device=dev)
    cr = routing.c()
    _check("moe_quantize_tokens_fp8", lib().moe_quantize_tokens_fp8(
        ctypes.byref(shape), _ptr(src), C, 1 if gather else 0, ctypes.byref(cr), _ptr(q), _ptr(s), _ptr(ws),
        ws.numel(), _stream(dev)))
    return q, s


def quantize_mxfp8(src, kind=QUANT_ROWS):
    """MXFP8 e4m3 codes (uint8) and E8M0 scale bytes (uint8) of a bf16
    tensor: kind QUANT_ROWS for [n0, n1] (blocks of 32 along rows; s [n0,
    n1/32]), QUANT_WEIGHT for [n0, n1, n2] (blocks of 32 along rows; s [n0,
    n1, n2/32]), QUANT_WEIGHT_T (blocks of 32 down columns, written
    transposed; q [n0, n2, n1], s [n0, n2, n1/32])."""
    dev = src.device
    if src.dtype != torch.bfloat16 or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 tensor")
    if kind == QUANT_ROWS:
        n0, n1 = src.shape
        n2 = 0
        qs = (n0, n1)
    else:
        n0, n1, n2 = src.shape
        qs = (n0, n1, n2) if kind == QUANT_WEIGHT else (n0, n2, n1)
    q = torch.empty(qs, dtype=torch.uint8, device=dev)
    s = torch.empty(qs[:-1] + (qs[-1] // 32,), dtype=torch.uint8, device=dev)
    _check("moe_quantize_mxfp8", lib().moe_quantize_mxfp8(kind, _ptr(src), n0, n1, n2, _ptr(q), _ptr(s),
                                                          _stream(dev)))
    return q, s


def quantize_tokens_mxfp8(src, routing: Routing, T, k, gather):
    """MXFP8 token-block codes q [C, 128 nblk] and scale bytes s [C, 4 nblk]
    of a weight-gradient operand (see moe_quantize_tokens_mxfp8)."""
    dev = src.device
    C = src.shape[1]
    E = routing.counts.numel()
    shape = make_shape(T, C, E, k, 128, torch.bfloat16)
    nblk = -(-T * k // 128) + E
    q = torch.zeros((C, 128 * nblk), dtype=torch.uint8, device=dev)
    s = torch.zeros((C, 4 * nblk), dtype=torch.uint8, device=dev)
    ws = torch.empty(workspace_size(shape, OP_ROUTE), dtype=torch.uint8, device=dev)
    cr = routing.c()
    _check("moe_quantize_tokens_mxfp8", lib().moe_quantize_tokens_mxfp8(
        ctypes.byref(shape), _ptr(src), C, 1 if gather else 0, ctypes.byref(cr), _ptr(q), _ptr(s), _ptr(ws),
        ws.numel(), _stream(dev)))
    return q, s
