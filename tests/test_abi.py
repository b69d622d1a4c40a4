"""The C-ABI library: it loads, exports every entry point include/moe.h
declares, and rejects bad arguments on the host before any HIP call (so
these run without a GPU: fake non-null device pointers are never touched)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from combine_top_route_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


# The calls of the boundary as the scope table names them (routing, forward,
# backward, the sizing queries, the standalone dispatch and combine, status
# strings), plus this library's status-returning sizes and timing hooks.
BOUNDARY = ("moe_route", "moe_forward", "moe_backward", "moe_workspace_bytes", "moe_saved_bytes",
            "moe_permute", "moe_combine", "moe_status_string")


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in BOUNDARY + ("moe_workspace_size", "moe_saved_size", "moe_last_error", "moe_profile_begin",
                         "moe_profile_end"):
        assert n in names


def test_sizing_calls_match_their_status_forms():
    """moe_workspace_bytes / moe_saved_bytes return the sizes the status
    forms report, and 0 (with a message) for a rejected shape or op."""
    lib = B.lib()
    for kw in (dict(), dict(dtype=torch.bfloat16, d=256, I=256, precision="fp8_block"),
               dict(dtype=torch.bfloat16, d=256, I=256, precision="mxfp8")):
        sh = _shape(**kw)
        for op in (B.OP_ROUTE, B.OP_FORWARD, B.OP_BACKWARD, B.OP_BACKWARD_RECOMPUTE):
            st, n = _status(sh, op)
            assert st == 0 and lib.moe_workspace_bytes(ctypes.byref(sh), op) == n > 0
        m = ctypes.c_size_t()
        assert lib.moe_saved_size(ctypes.byref(sh), ctypes.byref(m)) == 0
        assert lib.moe_saved_bytes(ctypes.byref(sh)) == m.value > 0
    bad = _shape(k=9)
    assert lib.moe_workspace_bytes(ctypes.byref(bad), B.OP_FORWARD) == 0
    assert b"k=9" in lib.moe_last_error()
    assert lib.moe_saved_bytes(ctypes.byref(bad)) == 0
    assert lib.moe_workspace_bytes(ctypes.byref(_shape()), 7) == 0
    assert lib.moe_workspace_bytes(None, 0) == 0


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = B.lib()
    for n in declared_functions():
        assert hasattr(lib, n)


def _shape(**kw):
    base = dict(T=64, d=64, E=8, k=2, I=128, dtype=torch.float32)
    base.update(kw)
    return B.make_shape(**base)


def _status(shape, op=B.OP_FORWARD):
    n = ctypes.c_size_t()
    return B.lib().moe_workspace_size(ctypes.byref(shape), op, ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw", [dict(T=0), dict(E=0), dict(E=1025), dict(k=0), dict(k=9),
                                dict(d=12), dict(I=4), dict(d=16392), dict(T=(1 << 24) + 1)])
def test_bad_shapes_rejected(kw):
    st, _ = _status(_shape(**kw))
    assert st == 1  # MOE_ERR_INVALID_ARGUMENT
    assert B.lib().moe_last_error().decode()


def test_bad_enums_rejected():
    s = _shape()
    s.dtype = 7
    assert _status(s)[0] == 1
    for bad in (-1.0, float("nan"), float("inf")):      # the SwiGLU clamp: 0 or a positive finite limit
        s = _shape()
        s.swiglu_limit = bad
        assert _status(s)[0] == 1 and b"swiglu_limit" in B.lib().moe_last_error()
    s = _shape(swiglu_limit=7.0)
    assert _status(s)[0] == 0
    for bad in (2, -1, 1 << 30):                        # flags: MOE_FLAG_PERSISTENT only
        s = _shape()
        s.flags = bad
        assert _status(s)[0] == 1 and b"flags" in B.lib().moe_last_error()
    assert _status(_shape(persistent=True))[0] == 0


def test_bf16_backward_workspace_holds_the_down_dgrad():
    # the bf16 backward keeps dH [R, 2I] and the down GEMM's data gradient
    # G [R, I] side by side, also when I is far above d
    for d, I in ((64, 2048), (2048, 64), (8, 16384)):
        st, w = _status(_shape(dtype=torch.bfloat16, d=d, I=I), op=B.OP_BACKWARD)
        R = 64 * 2
        assert st == 0 and w >= 2 * R * (2 * I + max(I, d)), (d, I, w)


def test_fp8_requirements():
    s = _shape(precision="fp8_block")                     # f32 storage
    assert _status(s)[0] == 2                            # MOE_ERR_UNSUPPORTED
    s = _shape(precision="fp8_block", dtype=torch.bfloat16, d=192, I=128)
    assert _status(s)[0] == 2
    # a valid fp8 shape: its workspaces hold the quantised operands besides the bf16 ones
    for op in (B.OP_FORWARD, B.OP_BACKWARD):
        st8, w8 = _status(_shape(precision="fp8_block", dtype=torch.bfloat16, d=256, I=128), op=op)
        st16, w16 = _status(_shape(dtype=torch.bfloat16, d=256, I=128), op=op)
        assert st8 == 0 and st16 == 0 and w8 > w16


def test_mxfp8_requirements_and_sizes():
    assert _status(_shape(precision="mxfp8"))[0] == 2                                  # f32 storage
    assert _status(_shape(precision="mxfp8", dtype=torch.bfloat16, d=192, I=128))[0] == 2
    bf = dict(dtype=torch.bfloat16, d=256, I=128)
    for op in (B.OP_FORWARD, B.OP_BACKWARD):
        stm, wm = _status(_shape(precision="mxfp8", **bf), op=op)
        st8, w8 = _status(_shape(precision="fp8_block", **bf), op=op)
        assert stm == 0 and st8 == 0 and wm >= w8
    # the saved buffer carries the transposed weights' scales: one byte per
    # 32 values (MX) rather than one float per 128 x 128 block
    sizes = {}
    for p in ("native", "fp8_block", "mxfp8"):
        n = ctypes.c_size_t()
        assert B.lib().moe_saved_size(ctypes.byref(_shape(precision=p, **bf)), ctypes.byref(n)) == 0
        sizes[p] = n.value
    E, d, I = 8, 256, 128
    assert sizes["fp8_block"] - sizes["native"] >= 3 * E * d * I            # both transposed codes
    assert sizes["mxfp8"] - sizes["fp8_block"] >= 3 * E * d * I // 32 - 1024   # 256-byte alignment


def test_fp8_bwd_sizes():
    """fp8_bwd: a bf16 forward (no weight codes saved), an fp8 backward that
    encodes the transposed weights in its own workspace."""
    bf = dict(dtype=torch.bfloat16, d=256, I=128)
    assert _status(_shape(precision="fp8_bwd"))[0] == 2                                # f32 storage
    assert _status(_shape(precision="fp8_bwd", **bf), op=B.OP_FORWARD) == \
        _status(_shape(**bf), op=B.OP_FORWARD)
    _, wb = _status(_shape(precision="fp8_bwd", **bf), op=B.OP_BACKWARD)
    _, w8 = _status(_shape(precision="fp8_block", **bf), op=B.OP_BACKWARD)
    assert wb >= w8 + 3 * 8 * 256 * 128
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    B.lib().moe_saved_size(ctypes.byref(_shape(precision="fp8_bwd", **bf)), ctypes.byref(n0))
    B.lib().moe_saved_size(ctypes.byref(_shape(**bf)), ctypes.byref(n1))
    assert n0.value == n1.value
    s = _shape(**bf)
    s.precision = 4
    assert _status(s)[0] == 1


def test_quantize_mxfp8_entry_points_validate():
    L = B.lib()
    q, sc = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert L.moe_quantize_mxfp8(B.QUANT_ROWS, None, 4, 128, 0, q, sc, None) == 1     # NULL src
    assert L.moe_quantize_mxfp8(5, FAKE, 4, 128, 0, q, sc, None) == 1                # unknown kind
    assert L.moe_quantize_mxfp8(B.QUANT_ROWS, FAKE, 4, 96, 0, q, sc, None) == 1      # 96 % 128
    assert L.moe_quantize_mxfp8(B.QUANT_WEIGHT_T, FAKE, 2, 128, 64, q, sc, None) == 1
    assert L.moe_quantize_mxfp8(B.QUANT_ROWS, FAKE, 4, 128, 0, q, ctypes.c_void_p((1 << 21) + 2),
                                None) == 1                                          # s alignment
    s = _shape(dtype=torch.bfloat16)
    r = B.MoeRouting(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_quantize_tokens_mxfp8(ctypes.byref(s), FAKE, 100, 1, ctypes.byref(r), q, sc, FAKE,
                                       1 << 30, None) == 1                          # C % 128
    assert L.moe_quantize_tokens_mxfp8(ctypes.byref(s), FAKE, 128, 1, ctypes.byref(r), q, sc, FAKE,
                                       0, None) == 3                                # workspace


def test_quantize_entry_points_validate():
    L = B.lib()
    q, sc = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert L.moe_quantize_fp8(B.QUANT_ROWS, None, 4, 128, 0, q, sc, None) == 1       # NULL src
    assert L.moe_quantize_fp8(9, FAKE, 4, 128, 0, q, sc, None) == 1                  # unknown kind
    assert L.moe_quantize_fp8(B.QUANT_ROWS, FAKE, 4, 100, 0, q, sc, None) == 1       # 100 % 128
    assert L.moe_quantize_fp8(B.QUANT_WEIGHT, FAKE, 2, 128, 96, q, sc, None) == 1    # 96 % 128
    assert L.moe_quantize_fp8(B.QUANT_ROWS, ctypes.c_void_p((1 << 20) + 8), 4, 128, 0, q, sc, None) == 1
    s = _shape(dtype=torch.bfloat16)
    r = B.MoeRouting(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_quantize_tokens_fp8(ctypes.byref(s), FAKE, 100, 1, ctypes.byref(r), q, sc, FAKE,
                                     1 << 30, None) == 1                            # C % 128
    assert L.moe_quantize_tokens_fp8(ctypes.byref(s), FAKE, 128, 1, ctypes.byref(r), q, sc, FAKE,
                                     0, None) == 3                                  # workspace
    s32 = _shape()
    assert L.moe_quantize_tokens_fp8(ctypes.byref(s32), FAKE, 128, 1, ctypes.byref(r), q, sc, FAKE,
                                     1 << 30, None) == 2                            # f32 storage


def test_workspace_sizes_grow_with_problem():
    _, a = _status(_shape(T=64))
    _, b = _status(_shape(T=640))
    assert 0 < a < b
    st, r = _status(_shape(), op=B.OP_ROUTE)
    assert st == 0 and 0 < r < a
    st, bw = _status(_shape(), op=B.OP_BACKWARD)
    assert st == 0 and bw > 0
    n = ctypes.c_size_t()
    s = _shape(T=10, k=2, I=16, dtype=torch.bfloat16)
    assert B.lib().moe_saved_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == 2 * 20 * 3 * 16


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation


def _routing(**null):
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k in null:
        setattr(r, k, None)
    return r


def test_forward_rejects_null_and_short_workspace_without_touching_the_gpu():
    lib = B.lib()
    s = _shape()
    r = _routing()
    args = lambda **o: [ctypes.byref(s), o.get("x", FAKE), ctypes.byref(o.get("r", r)), FAKE, FAKE,
                        o.get("out", FAKE), None, FAKE, o.get("ws", 1 << 40), None]
    assert lib.moe_forward(*args(x=None)) == 1
    assert lib.moe_forward(*args(out=None)) == 1
    assert lib.moe_forward(*args(r=_routing(row_of=1))) == 1
    assert lib.moe_forward(*args(ws=16)) == 3           # MOE_ERR_WORKSPACE
    assert "workspace" in lib.moe_last_error().decode()


def test_backward_rejects_dlogits_without_logits():
    lib = B.lib()
    s = _shape()
    r = _routing(logits=1)
    st = lib.moe_backward(ctypes.byref(s), FAKE, FAKE, ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE,
                          FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == 1
    assert "dlogits" in lib.moe_last_error().decode()


def test_misaligned_pointer_rejected():
    lib = B.lib()
    s = _shape()
    r = _routing()
    st = lib.moe_permute(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 2), ctypes.byref(r), FAKE, None)
    assert st == 1


def test_status_strings():
    lib = B.lib()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"


def test_route_noalloc_rejects_shapes_beyond_its_scratch():
    """Above 4 MiB of histograms (4 * ceil(T*k/1024) * E bytes) the
    no-allocation routing call refuses before touching the device."""
    lib = B.lib()
    sh = _shape(T=1 << 20, E=1024, k=2, d=64, I=64)   # 2048 chunks x 1024 experts x 4 B = 8 MiB
    r = B.MoeRouting(None, *([ctypes.c_void_p(16)] * 6))
    st = lib.moe_route_noalloc(ctypes.byref(sh), ctypes.byref(r), None)
    assert st == 2 and b"use moe_route with a workspace" in lib.moe_last_error()
    st = lib.moe_route_noalloc(ctypes.byref(_shape(k=9)), ctypes.byref(r), None)
    assert st == 1
    rn = B.MoeRouting(None, None, *([ctypes.c_void_p(16)] * 5))
    assert lib.moe_route_noalloc(ctypes.byref(_shape()), ctypes.byref(rn), None) == 1
