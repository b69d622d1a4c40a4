"""The shape contract that include/moe.h states, restated here from the
header's text and checked against the library's own validation on random
shapes (hypothesis): which shapes are rejected and with which status, and
what the sizing calls return for the accepted ones.  Host code only: no
call here reaches the GPU.
"""
import ctypes
import math

import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from combine_top_route_amd import binding as B

# the header's limits ("Limits checked by every call", moe_precision, moe_shape)
MAX_T, MAX_R, MAX_E, MAX_DI = 1 << 24, 1 << 27, 1024, 16384


def expected_status(T, d, E, k, I, dtype, ldt, prec, lim, flags):
    ok_ext = lambda n: 8 <= n <= MAX_DI and n % 8 == 0
    invalid = (not (1 <= T <= MAX_T) or not (1 <= E <= MAX_E) or not (1 <= k <= E) or T * k > MAX_R
               or not ok_ext(d) or not ok_ext(I) or dtype not in (0, 1) or ldt not in (0, 1)
               or prec not in (0, 1, 2, 3) or flags not in (0, 1)
               or not (lim == 0.0 or (lim > 0.0 and math.isfinite(lim))))
    if invalid:
        return 1  # MOE_ERR_INVALID_ARGUMENT
    if prec != 0 and (dtype != 1 or d % 128 or I % 128 or T * k * max(d, 2 * I) // 128 >= 1 << 31):
        return 2  # MOE_ERR_UNSUPPORTED
    return 0


def _sizes(shape):
    lib = B.lib()
    out = {}
    for op in (B.OP_ROUTE, B.OP_FORWARD, B.OP_BACKWARD, B.OP_BACKWARD_RECOMPUTE):
        n = ctypes.c_size_t(12345)
        st_ = lib.moe_workspace_size(ctypes.byref(shape), op, ctypes.byref(n))
        out[op] = (st_, n.value, lib.moe_workspace_bytes(ctypes.byref(shape), op))
    n = ctypes.c_size_t(12345)
    out["saved"] = (lib.moe_saved_size(ctypes.byref(shape), ctypes.byref(n)), n.value,
                    lib.moe_saved_bytes(ctypes.byref(shape)))
    return out


# each field mostly valid (so that whole shapes often are), sometimes not
extent = st.one_of(st.integers(1, 64).map(lambda x: 8 * x),
                   st.sampled_from([1000, 1536, 2048, 4096, 16376, 16384]),
                   st.sampled_from([-8, 0, 4, 12, 130, 16392, 1 << 20]))
shapes = st.tuples(
    st.one_of(st.integers(1, 5000), st.sampled_from([1 << 24]),
              st.sampled_from([-2, 0, (1 << 24) + 1, 1 << 25])),                        # T
    extent,                                                                               # d
    st.one_of(st.integers(1, 40), st.sampled_from([128, 1023, 1024]), st.sampled_from([-1, 0, 1025])),  # E
    st.one_of(st.integers(1, 12), st.sampled_from([64, 100, 1024]), st.sampled_from([-1, 0])),         # k
    extent,                                                                               # I
    st.sampled_from([0, 1, 1, -1, 2]), st.sampled_from([0, 1, 1, 2]),                     # dtypes
    st.sampled_from([0, 0, 1, 2, 3, -1, 4]),                                              # precision
    st.one_of(st.just(0.0), st.floats(min_value=2.0 ** -100, max_value=2.0 ** 127, width=32),
              st.floats(allow_nan=True, allow_infinity=True, width=32)),                  # swiglu_limit
    st.sampled_from([0, 0, 1, 2, -1]),                                                    # flags
)


@settings(max_examples=1500, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shapes)
def test_shape_validation_matches_the_header(args):
    T, d, E, k, I, dtype, ldt, prec, lim, flags = args
    s = B.MoeShape(T, d, E, k, I, dtype, ldt, prec, lim, flags)
    want = expected_status(T, d, E, k, I, dtype, ldt, prec, lim, flags)
    sizes = _sizes(s)
    for key, (status, n, nbytes) in sizes.items():
        assert status == want, (key, args, B.lib().moe_last_error().decode())
        if want:
            assert nbytes == 0, key  # the plain sizing calls return 0 on invalid input
            assert B.lib().moe_last_error().decode()
        else:
            assert n == nbytes and n > 0, key
    if want == 0:
        R, es = T * k, 4 if dtype == 0 else 2
        route, fwd, bwd, rec = (sizes[op][1] for op in (B.OP_ROUTE, B.OP_FORWARD, B.OP_BACKWARD,
                                                        B.OP_BACKWARD_RECOMPUTE))
        saved = sizes["saved"][1]
        # what the header promises the caller's buffers hold
        assert saved >= es * R * 3 * I  # H [R, 2I] and Aw [R, I]
        if prec == 0:
            assert saved == es * R * 3 * I
        assert fwd >= es * R * (d + I) and fwd % 256 == 0     # Y [R, d], Aw [R, I]
        assert bwd >= es * R * (2 * I + d) and bwd % 256 == 0  # dH [R, 2I], permuted dx [R, d]
        assert rec >= bwd + es * R * 3 * I                   # plus the recomputed H and Aw
        assert route % 256 == 0 and route <= fwd


@pytest.mark.parametrize("lim", [1e-30, 1.0, 3.0e38, float(torch.finfo(torch.float32).max)])
def test_every_positive_finite_limit_is_accepted(lim):
    s = B.make_shape(64, 64, 8, 2, 128, torch.bfloat16, swiglu_limit=lim)
    assert B.lib().moe_workspace_bytes(ctypes.byref(s), B.OP_FORWARD) > 0


# boundary shapes the random draw reaches rarely: the fp8 size limit at
# T*k = 2^27 (whose operand widest in K is 2I here), the largest extents
BOUNDARY = [
    (1 << 24, 1024, 128, 8, 1536, 1, 1, 1, 0.0, 0),   # fp8: 2^27 rows x 2I = 3072 -> unsupported
    (1 << 24, 1024, 128, 8, 896, 1, 1, 1, 0.0, 0),    # 2I = 1792 -> 14 * 2^27 < 2^31: accepted
    (1 << 24, 2048, 128, 8, 768, 1, 1, 2, 0.0, 0),    # d = 2048 -> 16 * 2^27 = 2^31: unsupported
    (1 << 24, 1024, 128, 8, 1536, 1, 1, 0, 0.0, 1),   # the same shape in bf16 is accepted
    (1, 16384, 1024, 1024, 16384, 0, 1, 0, 7.0, 0),   # largest extents, k = E
    ((1 << 27) // 1024, 8, 1024, 1024, 8, 1, 0, 0, 0.0, 0),  # T*k = 2^27 exactly
    ((1 << 27) // 1024 + 1, 8, 1024, 1024, 8, 1, 0, 0, 0.0, 0),  # one row too many
]


@pytest.mark.parametrize("args", BOUNDARY)
def test_boundary_shapes(args):
    s = B.MoeShape(*args)
    want = expected_status(*args)
    for key, (status, _, _) in _sizes(s).items():
        assert status == want, (key, args)
